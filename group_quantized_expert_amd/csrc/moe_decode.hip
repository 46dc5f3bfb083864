// moe_decode.hip -- single-token (decode) kernels and C entry points of libmoe.
//
// One MoE layer for one token is three kernels on one stream (one HIP-graph chain):
//   K1  router rows (E x H fp32) and the shared expert's gate/up rows with SwiGLU;
//       both depend only on the layer input.
//   K2  top-k of the router logits, recomputed by every block from the logits K1
//       wrote, then the routed experts' gate/up rows with SwiGLU (a2a-mcp.org "What
//       is Flash-MoE", deep dive 3: fused SwiGLU).
//   K3  down rows of the k routed + shared experts, with the weighted combine, the
//       sigmoid-gated shared expert and the residual add done in the same block
//       (deep dive 3: combine + residual + gating in one pass).
// The routing decision never leaves the device (the wiki summary's per-layer
// pipeline hands the expert work to the GPU without a host round trip).  No kernel
// uses atomics or cross-block waits: every dependency is a kernel boundary, and the
// values several blocks need (top-k, RMS statistics) are recomputed by each of them
// in the same order, so they agree bitwise.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "moe.h"
#include "moe_device.h"
#include "moe_host.h"
#include "moe_persist.h"

namespace moe {
namespace {

constexpr int kBlock = 512;  // threads of K1 blocks and of full K2 blocks (8 waves)
constexpr int kMaxBatch = 64;  // tokens per batched layer step

// Inputs in LDS are cut into chunks of CPC floats (the inputs of one 16-byte chunk of codes),
// each followed by 4 pad floats: a lane reads its chunk's inputs as consecutive float4, and
// without the pad the lanes of a wave, which read consecutive chunks, would all start on the
// same LDS banks.  Padded position of input c:
template <int CPC>
__device__ __forceinline__ int xpad(int c) { return (c / CPC) * (CPC + 4) + c % CPC; }
template <int CPC>
constexpr int xpad_size(int n) { return n / CPC * (CPC + 4); }

// N floats (x of one or more tokens) staged in LDS by a block of NT threads: loaded into
// registers first (issued before the weight loads, so waiting for x does not wait for the
// weights), then stored in the padded layout; only the first n floats are loaded (the rest read
// as zeros) when n < N.
// The registers are native 4-float vectors: float4 struct copies become memcpys that keep the
// array in memory (LDS or scratch) instead of registers.
template <int N, int NT>
struct XStage {
  typedef float v4f __attribute__((ext_vector_type(4)));
  static constexpr int kN = (N / 4 + NT - 1) / NT;  // float4 per thread
  v4f v[kN];
  // Buffer loads with the valid length as the buffer size: lanes past it read zeros, with no
  // branch per load (a branch per load made the compiler wait for the weight loads issued
  // after these before the x stores).
  __device__ __forceinline__ void load(const float* __restrict__ x, int n = N) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(x), (short)0, n * (int)sizeof(float), 0x00020000);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = (int)threadIdx.x + NT * i;
      v[i] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, idx * 16, 0, 0));
    }
  }
  // all N floats (zeros past the loaded length); xs holds the padded layout of N floats
  template <int CPC>
  __device__ __forceinline__ void store(float* xs) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int idx = (int)threadIdx.x + NT * i;
      if ((N / 4) % NT == 0 || idx < N / 4) *reinterpret_cast<v4f*>(xs + xpad<CPC>(4 * idx)) = v[i];
    }
  }
};

// ------------------------------------------------------------------------------------------
// K1: router logits + shared-expert gate/up/SwiGLU.
// Block b: router rows 2b, 2b+1 (one quarter row per wave) and h rows 4b..4b+3 of the
// shared expert (waves 0-3 gate rows, waves 4-7 up rows).  Router only: grid.y = token.  With
// the shared expert, each block loads its rows once and runs them over the T tokens, NTOK
// tokens at a time (their x staged together; the next group's x is loaded during this one's
// products).  Each token's arithmetic is the same whatever the grouping.
// ------------------------------------------------------------------------------------------
struct K1Args {
  const float* x;         // [T][H]
  int T;
  int norm;               // inputs are RMSNorm(x) (scale recomputed from x)
  float eps;
  const float* w_router;  // [E][H] or null
  int E;
  float* logits;          // [T][E]
  const uint8_t* shared;  // shared expert record or null
  int I;
  float* h_shared;        // token t's shared h at h_shared + t * h_stride
  int64_t h_stride;
  // shared-expert gate sg[t] = sigmoid(w_sg . x_t (* RMS scale)), computed by one extra block
  // (the last) when w_sg is not null; 1 when it is null
  const float* w_sg;      // [H] or null
  float* sg_ws;           // [T] or null (no gate output at all)
  float* sg_out;          // optional copy [T]
  // digit planes of the tokens' inputs for K2's products, built by dig_blocks trailing
  // blocks of the grid: token t's chunk c (inputs 32 c .. 32 c + 31) is the record at
  // xdig + (t H / 32 + c) kDigRec: its kDigPlanes planes, then (input sum, digit unit)
  uint4* xdig;            // [T][H / 32][kDigRec] or null
  float* xscale;          // [T]: 1 / sqrt(mean(x^2) + eps) of each token's input
  int dig_blocks;
  int dig_even_odd;       // q2 layers: planes hold the even, then the odd inputs of each 16
};

// Tokens per digit-plane block: 16 inputs per thread.
template <int H>
constexpr int k1_dig_tokens() { return kBlock / (H / 16); }

// A trailing K1 block: the digit planes (and RMS scale) of tokens blk * TPB .. + TPB - 1, one
// unit of 16 inputs per thread (the four units of a 64-input group in one lane quad).
template <bool EVEN_ODD, int H>
__device__ __forceinline__ void k1_digit_block(const K1Args& a, int blk) {
  constexpr int UT = H / 16, TPB = k1_dig_tokens<H>(), WPT = UT / 64;
  static_assert(kBlock % UT == 0 && UT % 64 == 0, "whole waves per token");
  __shared__ float wsq[kBlock / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tl = threadIdx.x / UT, u = threadIdx.x % UT;
  const int t = blk * TPB + tl;
  const bool ok = t < a.T;  // uniform per wave
  float v[16];
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 f = ok ? reinterpret_cast<const float4*>(a.x + (size_t)t * H + 16 * u)[i]
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    v[4 * i] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) sq = fmaf(v[i], v[i], sq);
  uint2 pl[kDigPlanes];
  float sum, unit;
  digit_unit16<EVEN_ODD, kDigPlanes>(v, pl, sum, unit);
  sum += dpp_f<kDppQuadXor1>(sum);  // the 32-input chunk of units u & ~1, u | 1
  if (ok) {
    uint4* rec = a.xdig + ((size_t)t * (H / 32) + (u >> 1)) * kDigRec;
    uint2* r2 = reinterpret_cast<uint2*>(rec);
#pragma unroll
    for (int k = 0; k < kDigPlanes; ++k) r2[2 * k + (u & 1)] = pl[k];
    if ((u & 1) == 0)
      rec[kDigPlanes] = make_uint4(__float_as_uint(sum), __float_as_uint(unit), 0u, 0u);
  }
  sq = seg_sum<64>(sq);
  if (lane == 0) wsq[wave] = sq;
  __syncthreads();
  if (ok && u == 0) {
    float ss = 0.f;
#pragma unroll
    for (int w = 0; w < WPT; ++w) ss += wsq[tl * WPT + w];
    a.xscale[t] = 1.f / sqrtf(ss / (float)H + a.eps);
  }
}

// The extra K1 block: shared-expert gates of all tokens, wave w taking tokens w, w + 8, ...
template <int H>
__device__ __forceinline__ void k1_gate_block(const K1Args& a) {
  constexpr int kV = H / 4 / 64;  // float4 per lane
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const float4* w4 = reinterpret_cast<const float4*>(a.w_sg);
  for (int t = wave; t < a.T; t += kBlock / 64) {
    const float4* x4 = reinterpret_cast<const float4*>(a.x + (size_t)t * H);
    float d = 0.f, ss = 0.f;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      const float4 xv = x4[lane + 64 * v], wv = w4[lane + 64 * v];
      d = fmaf(wv.x, xv.x, d);
      d = fmaf(wv.y, xv.y, d);
      d = fmaf(wv.z, xv.z, d);
      d = fmaf(wv.w, xv.w, d);
      ss = fmaf(xv.x, xv.x, ss);
      ss = fmaf(xv.y, xv.y, ss);
      ss = fmaf(xv.z, xv.z, ss);
      ss = fmaf(xv.w, xv.w, ss);
    }
    d = seg_sum<64>(d);
    ss = seg_sum<64>(ss);
    const float xscale = a.norm ? 1.f / sqrtf(ss / (float)H + a.eps) : 1.f;
    if (lane == 0) {
      const float g = sigmoidf_acc(d * xscale);
      a.sg_ws[t] = g;
      if (a.sg_out) a.sg_out[t] = g;
    }
  }
}

constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i of each 8 <- lane 7 - i

// sum over aligned groups of 8 lanes, in every lane of the group
__device__ __forceinline__ float sum8(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v;
}

// The 16-byte chunk's codes as floats in element order (each exact, times 2^-9).
template <int BITS>
__device__ __forceinline__ void codes_f32(const uint4 c, float (&f)[128 / BITS]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (BITS == 4) {
      const uint32_t lo = w[d] & 0x0F0F0F0Fu, hi = (w[d] >> 4) & 0x0F0F0F0Fu;
      float* o = f + 8 * d;
      codes2<false>(lo, o[0], o[2]);
      codes2<true>(lo, o[4], o[6]);
      codes2<false>(hi, o[1], o[3]);
      codes2<true>(hi, o[5], o[7]);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t b = (w[d] >> (2 * m)) & 0x03030303u;  // elements 16 d + 4 j + m
        float* o = f + 16 * d + m;
        codes2<false>(b, o[0], o[4]);
        codes2<true>(b, o[8], o[12]);
      }
    }
  }
}

// The shared-expert rows of a K1 block, gate rows hi0 .. hi0 + 3 then the up rows, split over
// the block's 8 waves by input: wave w takes the w-th eighth of the inputs of all 8 rows, lane l
// row l / 8 and chunks (l % 8) + kLR p of that eighth (for small H only the first kLR lanes of
// each row work).  A wave so reads an eighth of each token's input from LDS, and converts each
// chunk's codes once for all the tokens staged together.
template <int BITS, int H>
struct SharedSlice {
  using G = Geo<BITS, H>;
  static constexpr int CPC = G::kCodesPerChunk;
  static constexpr int kCS = H / 8 / CPC;        // chunks of each row in a wave's eighth
  static constexpr int kLR = kCS < 8 ? kCS : 8;  // working lanes per row
  static constexpr int kP = kCS / kLR;           // chunks per working lane
  static_assert(kCS >= 1 && kCS % kLR == 0, "");
  uint4 q[kP];
  uint16_t s[kP], b[kP];
  int chunk[kP];
  bool act;

  // rows hi0 .. hi0 + 3 of the gate and up matrices of the record at rec (I rows each)
  __device__ __forceinline__ void load(const uint8_t* __restrict__ rec, int I, int hi0, int wave,
                                       int lane) {
    const int rr = lane >> 3, hi = hi0 + (rr & 3);
    const uint8_t* m = rec + (rr < 4 ? 0 : matrix_rec_bytes<BITS>(I, H));
    const uint8_t* codes = m + (size_t)hi * G::kRowBytes;
    const uint16_t* scale = reinterpret_cast<const uint16_t*>(m + (size_t)I * G::kRowBytes);
    const uint16_t* bias = scale + (size_t)I * G::kGroupsPerRow;
    act = (lane & 7) < kLR;
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      chunk[p] = wave * kCS + (lane & 7) % kLR + kLR * p;
      q[p] = ld_nt_u4(codes + chunk[p] * 16);
      const int gi = hi * G::kGroupsPerRow + chunk[p] / G::kChunksPerGroup;
      s[p] = __builtin_nontemporal_load(scale + gi);
      b[p] = __builtin_nontemporal_load(bias + gi);
    }
  }

  // Makes the loaded values opaque to the optimizer at this point, so that work on them alone
  // (code conversion, scale unpacking) is not hoisted out of the loop over token groups to
  // where it would wait for the loads before the first group's inputs are staged.
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      uint32_t sb = (uint32_t)s[p] | ((uint32_t)b[p] << 16);
      asm volatile("" : "+v"(q[p].x), "+v"(q[p].y), "+v"(q[p].z), "+v"(q[p].w), "+v"(sb));
      s[p] = (uint16_t)sb;
      b[p] = (uint16_t)(sb >> 16);
    }
  }

  // This lane's partial of its row for tokens 0 .. ng - 1 of the group: token tt's padded
  // inputs at xs + tt xstride, its chunk sums at xsum + tt kCh.  The codes are converted once;
  // one token's inputs are live at a time.
  template <int NTOK>
  __device__ __forceinline__ void products(const float* __restrict__ xs, int xstride,
                                           const float* __restrict__ xsum, int kCh, int ng,
                                           float (&acc)[NTOK]) const {
    float cf[kP][CPC], sc[kP], bc[kP];
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      codes_f32<BITS>(q[p], cf[p]);
      sc[p] = bf16f(s[p]) * kCodeUnit;
      bc[p] = bf16f(b[p]);
    }
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
      acc[tt] = 0.f;
      if (tt >= ng) continue;
#pragma unroll
      for (int p = 0; p < kP; ++p) {
        const float4* x4 = reinterpret_cast<const float4*>(xs + tt * xstride + chunk[p] * (CPC + 4));
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int v = 0; v < CPC / 4; ++v) {
          const float4 f = x4[v];
          d0 = fmaf(cf[p][4 * v], f.x, d0);
          d1 = fmaf(cf[p][4 * v + 1], f.y, d1);
          d0 = fmaf(cf[p][4 * v + 2], f.z, d0);
          d1 = fmaf(cf[p][4 * v + 3], f.w, d1);
        }
        acc[tt] += sc[p] * (d0 + d1) + bc[p] * xsum[tt * kCh + chunk[p]];
      }
      if (!act) acc[tt] = 0.f;
      issue_fence();  // the next token's inputs are read only now
    }
  }
};

template <int BITS, int H, bool SHARED, int NTOK>
__global__ __launch_bounds__(kBlock) void k1_kernel(K1Args a) {
  using G = Geo<BITS, H>;
  constexpr int kQ = H / 4 / 4 / 64;  // float4 per lane in a quarter row
  static_assert(SHARED || NTOK == 1, "router-only blocks take one token (grid.y)");
  // with the shared expert, NTOK == 1 is launched for a single token only
  constexpr int CPC = G::kCodesPerChunk;
  constexpr int kXP = xpad_size<CPC>(H);  // padded floats per token
  __shared__ __align__(16) float xs[NTOK][kXP];
  constexpr int kCh = H / CPC;            // chunks per token
  __shared__ float part[NTOK][8];
  __shared__ float psh[NTOK][8][8];       // shared rows: [token][wave][row] partials
  __shared__ float xsum_s[NTOK * kCh];    // per-chunk input sums of the group's tokens
  __shared__ float sq_s[NTOK * kCh];      // per-chunk sums of squares
  __shared__ float xscale_s[NTOK];
  const int nbx = (int)gridDim.x - a.dig_blocks;  // blocks before the digit-plane blocks
  if ((int)blockIdx.x >= nbx) {
    if (blockIdx.y == 0) {
      if (a.dig_even_odd)
        k1_digit_block<true, H>(a, (int)blockIdx.x - nbx);
      else
        k1_digit_block<false, H>(a, (int)blockIdx.x - nbx);
    }
    return;
  }
  if (a.sg_ws && (int)blockIdx.x == nbx - 1) {
    if (blockIdx.y != 0) return;
    if (a.w_sg) {
      k1_gate_block<H>(a);
    } else if (threadIdx.x < a.T) {
      a.sg_ws[threadIdx.x] = 1.f;
      if (a.sg_out) a.sg_out[threadIdx.x] = 1.f;
    }
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t_first = SHARED ? 0 : blockIdx.y;
  const int T = SHARED && NTOK > 1 ? a.T : 1;  // one-token blocks are launched for T == 1 only

  XStage<NTOK * H, kBlock> xv;
  xv.load(a.x + (size_t)t_first * H, (T < NTOK ? T : NTOK) * H);
  issue_fence();
  // router quarter row r (4 waves per row); rows past E load row E-1 and are not written
  const int r = blockIdx.x * 2 + (wave >> 2);
  const int q = wave & 3;
  const bool do_router = r < a.E;
  float4 wv[kQ];
  {
    const float* wr = a.w_router + (size_t)(do_router ? r : a.E - 1) * H + q * (H / 4);
#pragma unroll
    for (int j = 0; j < kQ; ++j) wv[j] = ld_nt_f4(wr + 4 * (lane + 64 * j));
  }
  // shared expert: h rows hi0 .. hi0 + 3 (blocks past I load the last four rows and write
  // nothing)
  const int hi0 = blockIdx.x * 4;
  const bool do_shared = SHARED && hi0 < a.I;
  SharedSlice<BITS, H> sh;
  if constexpr (SHARED) sh.load(a.shared, a.I, do_shared ? hi0 : a.I - 4, wave, lane);
  issue_fence();
  // One group of up to NTOK tokens.  The first group runs outside the loop over the others, so
  // that its wait for x is not merged with the later groups' (which would make it wait for the
  // weight loads too).
  auto group = [&](const int g0) {
    const int ng = T - g0 < NTOK ? T - g0 : NTOK;
    if (g0) __syncthreads();  // the previous group's xs, part and psh have been read
    xv.template store<CPC>(&xs[0][0]);
    if (g0 + NTOK < T) {
      const int nn = T - g0 - NTOK < NTOK ? T - g0 - NTOK : NTOK;
      xv.load(a.x + (size_t)(t_first + g0 + NTOK) * H, nn * H);
    }
    __syncthreads();
    // Per-chunk input sums and RMS scales of the group's tokens, once per block (every wave
    // needs the same ones): thread i takes chunk i of the group, summing in element order.
    if (SHARED || a.norm) {
      for (int i = threadIdx.x; i < ng * kCh; i += kBlock) {
        const float* src = &xs[0][0] + i * (CPC + 4);
        float sm = 0.f, sq = 0.f;
#pragma unroll
        for (int c = 0; c < CPC; c += 4) {
          const float4 v = *reinterpret_cast<const float4*>(src + c);
          sm += v.x;
          sm += v.y;
          sm += v.z;
          sm += v.w;
          sq = fmaf(v.x, v.x, sq);
          sq = fmaf(v.y, v.y, sq);
          sq = fmaf(v.z, v.z, sq);
          sq = fmaf(v.w, v.w, sq);
        }
        xsum_s[i] = sm;
        sq_s[i] = sq;
      }
      __syncthreads();
      if (a.norm && wave < ng) {  // wave tt: RMS scale of token tt
        float ss = 0.f;
        for (int c = lane; c < kCh; c += 64) ss += sq_s[wave * kCh + c];
        ss = seg_sum<64>(ss);
        if (lane == 0) xscale_s[wave] = 1.f / sqrtf(ss / (float)H + a.eps);
      }
      __syncthreads();
    }
    float xscale[NTOK];
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
      if (tt >= ng) break;
      xscale[tt] = a.norm ? xscale_s[tt] : 1.f;
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        const float4 xq = *reinterpret_cast<const float4*>(
            xs[tt] + xpad<CPC>(q * (H / 4) + 4 * (lane + 64 * j)));
        acc = fmaf(wv[j].x, xq.x, acc);
        acc = fmaf(wv[j].y, xq.y, acc);
        acc = fmaf(wv[j].z, xq.z, acc);
        acc = fmaf(wv[j].w, xq.w, acc);
      }
      acc = seg_sum<64>(acc);
      if (lane == 0) part[tt][wave] = acc;
    }
    if constexpr (SHARED) {
      sh.opaque();  // keeps the codes' conversion inside the group, after the inputs are staged
      float acc[NTOK];
      sh.template products<NTOK>(&xs[0][0], kXP, xsum_s, kCh, ng, acc);
#pragma unroll
      for (int tt = 0; tt < NTOK; ++tt) {
        if (tt >= ng) break;
        const float v = sum8(acc[tt]);
        if ((lane & 7) == 0) psh[tt][wave][lane >> 3] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < NTOK; ++tt) {
      if (tt >= ng) break;
      const int t = t_first + g0 + tt;
      if (do_router && q == 0 && lane == 0)  // waves wave..wave+3 hold the four quarters of row r
        a.logits[(size_t)t * a.E + r] =
            (((part[tt][wave] + part[tt][wave + 1]) + part[tt][wave + 2]) + part[tt][wave + 3]) *
            xscale[tt];
    }
    if (SHARED && do_shared && (int)threadIdx.x < 4 * ng) {
      // h of row hi0 + i for token i / 4: the eight waves' partials of its gate and up rows
      const int tt = threadIdx.x >> 2, i = threadIdx.x & 3;
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        g += psh[tt][w][i];
        u += psh[tt][w][4 + i];
      }
      const float xsc = a.norm ? xscale_s[tt] : 1.f;
      a.h_shared[(size_t)(t_first + g0 + tt) * a.h_stride + hi0 + i] =
          siluf_acc(g * xsc) * (u * xsc);
    }
  };
  group(0);
  for (int g0 = NTOK; g0 < T; g0 += NTOK) group(g0);
}

// ------------------------------------------------------------------------------------------
// K2: routed gate/up/SwiGLU.  With R = rows per wave pass, a block of WAVES waves covers
// 2 R WAVES h rows of one slot: wave w handles rows base + 2Rw + sub and base + 2Rw + R + sub
// (sub = lane's row within the pass).  Few slots take small blocks, so that the launch still
// spreads over the chip.  Slots come from the top-k of each token's router logits (slot j is
// rank j % k of token j / k; each block recomputes the top-k) or from an id array (one token).
// ------------------------------------------------------------------------------------------
struct K2Args {
  const float* x;          // [T][H]
  int norm;
  float eps;
  const float* logits;     // [T][E]: top-k mode when not null
  int E, k;
  const int32_t* ids_in;   // id mode: [n]
  int n;                   // slots processed: T k in top-k mode
  const uint8_t* base;
  int64_t slot_bytes;
  int n_slots_total;
  int I;
  float* h;                // slot j's h at h + hrow(j) I
  int h_per_token;         // top-k mode: h rows per token (k, plus one for a shared slot)
  // top-k mode: token t's routing, written by the first block of its rank-0 slot
  int32_t* ids_ws;         // [T][h_per_token] (shared slot in column k when shared_slot >= 0)
  float* w_ws;             // [T][k]
  int shared_slot;
  int32_t* ids_out;        // optional copies: [T][h_per_token], [T][k]
  float* w_out;
  int32_t* ids_trace;      // optional [T][k]
  int32_t* dev_err;
  // top-k mode: the tokens' digit planes and RMS scales from K1 (the products then run on
  // v_dot8_i32_i4), or null (fp32 products on x)
  const uint4* xdig;
  const float* xscale;
  // top-k mode: the routing already written to ids_ws / w_ws by route_kernel (then K2 blocks
  // read their ids instead of each recomputing the token's top-k)
  int routed;
};

template <int BITS, int H, int WAVES>
constexpr int k2_rows_per_block() { return 2 * WAVES * Geo<BITS, H>::kRowsPerWave; }

// Token t's routing into the workspace (for K3) and the optional copies; K1 writes the shared
// gate.
__device__ __forceinline__ void write_route(const K2Args& a, int t, const int (&ids)[kMaxTopK],
                                            const float (&w)[kMaxTopK]) {
  const size_t ti = (size_t)t * a.h_per_token, tw = (size_t)t * a.k;
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    if (s >= a.k) break;
    a.ids_ws[ti + s] = ids[s];
    a.w_ws[tw + s] = w[s];
    if (a.ids_out) a.ids_out[ti + s] = ids[s];
    if (a.w_out) a.w_out[tw + s] = w[s];
    if (a.ids_trace) a.ids_trace[tw + s] = ids[s];
  }
  if (a.shared_slot >= 0) {
    a.ids_ws[ti + a.k] = a.shared_slot;
    if (a.ids_out) a.ids_out[ti + a.k] = a.shared_slot;
  }
}

// The routing of token blockIdx.x (one wave), for K2 launches over many tokens.
__global__ __launch_bounds__(64) void route_kernel(K2Args a) {
  const int t = blockIdx.x;
  int ids[kMaxTopK];
  float vals[kMaxTopK], w[kMaxTopK];
  wave_topk(a.logits + (size_t)t * a.E, a.E, a.k, ids, vals, w);
  if (threadIdx.x == 0) write_route(a, t, ids, w);
}

// At most 128 VGPRs for q4 (four waves per SIMD: four 4-wave or two 8-wave blocks per CU, so
// that the latency of one block's top-k and first loads overlaps the others' streaming); q2,
// whose 64-code chunks need more registers, is held to three waves per SIMD.
template <int BITS, int H, int WAVES, bool DIG>
__global__ __launch_bounds__(64 * WAVES, BITS == 4 ? 4 : 3) void k2_kernel(K2Args a) {
  using G = Geo<BITS, H>;
  constexpr int R = G::kRowsPerWave;
  constexpr int kRB = k2_rows_per_block<BITS, H, WAVES>();
  constexpr int CPC = G::kCodesPerChunk;
  // the token's input, or its digit-plane records (H / 32 of 4 kDigRec floats' size), padded
  constexpr int kXN = DIG ? H / 32 * 4 * kDigRec : H;  // floats staged
  constexpr int kXC = DIG ? 4 * kDigRec : CPC;         // floats per padded unit
  constexpr int kXS = xpad_size<kXC>(kXN);
  __shared__ __align__(16) float xs[kXS];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int blocks_per_slot = a.I / kRB;
  const int j = blockIdx.x / blocks_per_slot;
  const bool topk_mode = a.logits != nullptr;
  const int t = topk_mode ? j / a.k : 0;
  const int rank = topk_mode ? j % a.k : j;
  XStage<kXN, 64 * WAVES> xv;
  xv.load(DIG ? reinterpret_cast<const float*>(a.xdig + (size_t)t * (H / 32) * kDigRec)
              : a.x + (size_t)t * H);
  LaneRow<BITS, H> lr;
  lr.set_lane(lane);
  const int i0 = (blockIdx.x % blocks_per_slot) * kRB + 2 * R * wave + lr.sub;
  const int i1 = i0 + R;

  // top-k of the token's logits on wave 0 only (the other waves would compute the same), the
  // block's slot id passed on through LDS; or the id route_kernel wrote
  __shared__ int s_e;
  int e;
  // wave 0 of the first block of a token's rank-0 slot writes the token's routing for K3
  const bool route_out = topk_mode && rank == 0 && blockIdx.x % blocks_per_slot == 0 && wave == 0;
  if (topk_mode && a.routed) {
    e = a.ids_ws[(size_t)t * a.h_per_token + rank];
  } else if (topk_mode) {
    if (wave == 0) {
      int ids[kMaxTopK];
      float vals[kMaxTopK], w[kMaxTopK];
      wave_topk(a.logits + (size_t)t * a.E, a.E, a.k, ids, vals, w);
      e = ids[0];
#pragma unroll
      for (int s = 1; s < kMaxTopK; ++s)
        if (s == rank) e = ids[s];
      if (lane == 0) s_e = e;
      if (route_out && lane == 0) write_route(a, t, ids, w);
    }
    __syncthreads();
    e = s_e;
  } else {
    e = a.ids_in[j];
  }
  const bool valid = e >= 0 && e < a.n_slots_total;  // invalid ids load slot 0, write zeros
  RowLoad<BITS, H> lg0, lg1, lu0, lu1;
  const size_t mat = matrix_rec_bytes<BITS>(a.I, H);
  {
    const uint8_t* rec = a.base + (size_t)(valid ? e : 0) * a.slot_bytes;
    lg0.load(rec, a.I, i0, lr);
    lg1.load(rec, a.I, i1, lr);
    lu0.load(rec + mat, a.I, i0, lr);
    lu1.load(rec + mat, a.I, i1, lr);
  }
  issue_fence();
  xv.template store<kXC>(xs);
  __syncthreads();

  float g0 = 0.f, g1 = 0.f, u0 = 0.f, u1 = 0.f, xscale = 1.f;
  if constexpr (DIG) {
    // Each pass's chunk records from LDS (the padded layout keeps the records of consecutive
    // lanes on different banks): the digit planes, then the input sum and unit.
    constexpr int NR = RowLoad<BITS, H>::kRecs;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      uint4 pl[NR][kDigPlanes];
      float xsum[NR], unit[NR];
#pragma unroll
      for (int h = 0; h < NR; ++h) {
        const uint4* rec = reinterpret_cast<const uint4*>(xs + (lr.chunk[p] * NR + h) * (kXC + 4));
#pragma unroll
        for (int k = 0; k < kDigPlanes; ++k) pl[h][k] = rec[k];
        const uint4 aux = rec[kDigPlanes];
        xsum[h] = __uint_as_float(aux.x);
        unit[h] = __uint_as_float(aux.y);
      }
      g0 += lg0.term_int(p, pl, xsum, unit);
      g1 += lg1.term_int(p, pl, xsum, unit);
      u0 += lu0.term_int(p, pl, xsum, unit);
      u1 += lu1.term_int(p, pl, xsum, unit);
      issue_fence();  // the next pass's records are read only now
    }
    if (a.norm) xscale = a.xscale[t];
  } else {
    // The lane's inputs pass by pass from LDS, each pass used by the wave's four rows at once
    // (so only one pass of inputs is live); chunk sums and sums of squares are accumulated in
    // the same element order as LaneRow and RowLoad::partial use.
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      float xp[CPC];
      const float4* src = reinterpret_cast<const float4*>(xs + lr.chunk[p] * (CPC + 4));
#pragma unroll
      for (int v = 0; v < CPC / 4; ++v) {
        const float4 f = src[v];
        xp[4 * v] = f.x;
        xp[4 * v + 1] = f.y;
        xp[4 * v + 2] = f.z;
        xp[4 * v + 3] = f.w;
      }
      float xsum = 0.f;
#pragma unroll
      for (int c = 0; c < CPC; ++c) xsum += xp[c];
#pragma unroll
      for (int c = 0; c < CPC; ++c) ss = fmaf(xp[c], xp[c], ss);
      g0 += lg0.term(p, xp, xsum);
      g1 += lg1.term(p, xp, xsum);
      u0 += lu0.term(p, xp, xsum);
      u1 += lu1.term(p, xp, xsum);
      issue_fence();  // the next pass's inputs are read only now
    }
    if (a.norm) xscale = 1.f / sqrtf(seg_sum<G::kLanesPerRow>(ss) / (float)H + a.eps);
  }
  g0 = seg_sum<G::kLanesPerRow>(g0) * xscale;
  g1 = seg_sum<G::kLanesPerRow>(g1) * xscale;
  u0 = seg_sum<G::kLanesPerRow>(u0) * xscale;
  u1 = seg_sum<G::kLanesPerRow>(u1) * xscale;
  if ((lane % G::kLanesPerRow) == 0) {
    const size_t hrow = topk_mode ? (size_t)t * a.h_per_token + rank : (size_t)j;
    float* hj = a.h + hrow * a.I;
    hj[i0] = valid ? siluf_acc(g0) * u0 : 0.f;
    hj[i1] = valid ? siluf_acc(g1) * u1 : 0.f;
  }
  if (!valid && lane == 0 && a.dev_err) *a.dev_err = 1;
}

// ------------------------------------------------------------------------------------------
// K3: down rows for the n slots of a token over kDownRows output rows per block (grid.y =
// token); slot j has KW waves, each taking an equal share of the rows (few slots take more
// waves per slot, so that a block still keeps several waves of loads in flight).
// Mode Y (y != null, one token): y[j][r] = deq(W_down[ids[j]]) h[j].
// Mode combine: out[t][r] = residual[t][r] + sum_j coef_j * y_j[r], coef_j = route_w[t][j] for
// j < n_routed, else sg[t] (or 1 when sg is null).
// ------------------------------------------------------------------------------------------
struct K3Args {
  const uint8_t* base;
  int64_t slot_bytes;
  int n_slots_total;
  const int32_t* ids;    // token t's n ids at ids + t n
  int n;
  const float* h;        // token t's slot j at h + (t n + j) I
  int H;
  float* y;              // mode Y
  const float* residual; // [T][H]
  const float* route_w;  // [T][n_routed]
  int n_routed;
  const float* sg;       // [T] or null
  float* out;            // [T][H]
  int32_t* dev_err;
};

template <int BITS, int I>
constexpr int k3_row_blocks() { return kDownRows / Geo<BITS, I>::kRowsPerWave; }

template <int BITS, int I, int KW>
__global__ __launch_bounds__(64 * (kMaxTopK + 1)) void k3_kernel(K3Args a) {
  using G = Geo<BITS, I>;
  constexpr int kRB = k3_row_blocks<BITS, I>() / KW;  // row blocks per wave
  static_assert(kDownRows % G::kRowsPerWave == 0 && k3_row_blocks<BITS, I>() % KW == 0, "");
  const int lane = threadIdx.x & 63;
  const int wi = threadIdx.x >> 6;
  const int j = wi / KW, qw = wi % KW;
  const int t = blockIdx.y;
  const int r0 = blockIdx.x * kDownRows;
  __shared__ float ybuf[kMaxTopK + 1][kDownRows];

  const int e = a.ids[(size_t)t * a.n + j];
  const bool valid = e >= 0 && e < a.n_slots_total;
  LaneRow<BITS, I> lr;
  lr.set_lane(lane);
  lr.load_x(a.h + ((size_t)t * a.n + j) * I);
  issue_fence();
  RowLoad<BITS, I> ld[kRB];
  {
    // invalid ids load slot 0 and contribute zeros
    const uint8_t* rec = a.base + (size_t)(valid ? e : 0) * a.slot_bytes +
                         2 * matrix_rec_bytes<BITS>(I, a.H);
#pragma unroll
    for (int b = 0; b < kRB; ++b)
      ld[b].load(rec, a.H, r0 + (qw * kRB + b) * G::kRowsPerWave + lr.sub, lr);
  }
  issue_fence();
  lr.finish();
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    const float v = seg_sum<G::kLanesPerRow>(ld[b].partial(lr));
    if ((lane % G::kLanesPerRow) == 0)
      ybuf[j][(qw * kRB + b) * G::kRowsPerWave + lr.sub] = valid ? v : 0.f;
  }
  if (!valid && lane == 0 && qw == 0 && a.dev_err) *a.dev_err = 1;
  __syncthreads();
  if (a.y) {
    for (int i = threadIdx.x; i < a.n * kDownRows; i += blockDim.x) {
      const int jj = i / kDownRows, rr = i % kDownRows;
      a.y[(size_t)jj * a.H + r0 + rr] = ybuf[jj][rr];
    }
    return;
  }
  if (threadIdx.x < kDownRows) {
    const int r = r0 + threadIdx.x;
    float o = a.residual[(size_t)t * a.H + r];
    for (int jj = 0; jj < a.n; ++jj) {
      const float c = jj < a.n_routed ? a.route_w[(size_t)t * a.n_routed + jj]
                                      : (a.sg ? a.sg[t] : 1.f);
      o = fmaf(c, ybuf[jj][threadIdx.x], o);
    }
    a.out[(size_t)t * a.H + r] = o;
  }
}

// xn = x / sqrt(mean(x^2) + eps), one block per row of H (row blockIdx.x).  Each thread
// writes only the elements it read, after the block-wide sum, so xn may equal x.
__global__ __launch_bounds__(1024) void rmsnorm_kernel(const float* x, int H, float eps,
                                                      float* xn) {
  __shared__ float red[16];
  x += (size_t)blockIdx.x * H;
  xn += (size_t)blockIdx.x * H;
  constexpr int kKeep = 8;  // the first 8 * blockDim.x elements stay in registers
  float v[kKeep];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kKeep; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    v[j] = i < H ? x[i] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kKeep; ++j) s = fmaf(v[j], v[j], s);
  for (int i = threadIdx.x + kKeep * blockDim.x; i < H; i += blockDim.x) s = fmaf(x[i], x[i], s);
  s = block_sum(s, red);
  const float sc = 1.f / sqrtf(s / (float)H + eps);
#pragma unroll
  for (int j = 0; j < kKeep; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    if (i < H) xn[i] = v[j] * sc;
  }
  for (int i = threadIdx.x + kKeep * blockDim.x; i < H; i += blockDim.x) xn[i] = x[i] * sc;
}

// Router top-k for T tokens, one wave per token (router_topk entry point).
__global__ __launch_bounds__(64) void topk_kernel(const float* __restrict__ logits, int E, int k,
                                                  const float* __restrict__ x,
                                                  const float* __restrict__ w_sg, int H,
                                                  int32_t* ids, int ld_ids, float* weights,
                                                  float* sg) {
  const int t = blockIdx.x;
  int id[kMaxTopK];
  float vals[kMaxTopK], w[kMaxTopK];
  wave_topk(logits + (size_t)t * E, E, k, id, vals, w);
  float g = 0.f;
  if (w_sg && sg) {
    for (int c = threadIdx.x; c < H; c += 64) g = fmaf(w_sg[c], x[(size_t)t * H + c], g);
    g = sigmoidf_acc(seg_sum<64>(g));
  }
  if (threadIdx.x == 0) {
    for (int s = 0; s < k; ++s) {
      ids[(size_t)t * ld_ids + s] = id[s];
      weights[(size_t)t * k + s] = w[s];
    }
    if (w_sg && sg) sg[t] = g;
  }
}

// ------------------------------------------------------------------------------------------
// Generic quantized matvec y = deq(W) x (building block export).
// ------------------------------------------------------------------------------------------
template <int BITS, int C>
__global__ __launch_bounds__(256) void qgemv_kernel(const uint8_t* __restrict__ rec, int R,
                                                    const float* __restrict__ x,
                                                    float* __restrict__ y) {
  using G = Geo<BITS, C>;
  constexpr int U = 4;
  // x is staged once per workgroup: every wave needs all of it, and reading it from global
  // memory per wave costs more L1 misses than the wave's own weight rows at C = 8192.  Each
  // chunk's inputs are followed by 4 pad floats so that lanes reading consecutive chunks
  // start on different LDS banks.
  constexpr int kStride = G::kCodesPerChunk + 4;
  __shared__ __align__(16) float xs[G::kChunksPerRow * kStride];
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (blockDim.x >> 6);
  LaneRow<BITS, C> lr;
  lr.set_lane(lane);
  const int nrb = (R + G::kRowsPerWave - 1) / G::kRowsPerWave;
  RowLoad<BITS, C> ld[U];
  int row[U];
  auto issue = [&](int b0) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      row[i] = (b0 + i) * G::kRowsPerWave + lr.sub;
      if (b0 + i < nrb && row[i] < R) ld[i].load(rec, R, row[i], lr);
    }
  };
  int b0 = wave * U;
  issue(b0);  // the first rows are in flight while x is staged
  for (int i = threadIdx.x; i < C / 4; i += blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(x)[i];
    const int c = 4 * i;
    *reinterpret_cast<float4*>(&xs[(c / G::kCodesPerChunk) * kStride + c % G::kCodesPerChunk]) = v;
  }
  __syncthreads();
  lr.load_x(xs, kStride);
  lr.finish();
  for (; b0 < nrb; b0 += nwaves * U) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (b0 + i >= nrb) break;
      const bool ok = row[i] < R;
      float v = seg_sum<G::kLanesPerRow>(ok ? ld[i].partial(lr) : 0.f);
      if (ok && (lane % G::kLanesPerRow) == 0) y[row[i]] = v;
    }
    if (b0 + nwaves * U < nrb) issue(b0 + nwaves * U);
  }
}

// Standalone combine (one block) with optional two-pass RMSNorm.
__global__ __launch_bounds__(1024) void combine_kernel(const float* __restrict__ residual,
                                                       const float* __restrict__ y,
                                                       const float* __restrict__ w, int k,
                                                       const float* __restrict__ sg,
                                                       float* out, float* __restrict__ out_norm,
                                                       float eps, int H) {
  __shared__ float red[16];
  const float g = sg ? *sg : 1.f;
  float ss = 0.f;
  for (int c = threadIdx.x; c < H; c += blockDim.x) {
    float o = residual[c];
    for (int j = 0; j < k; ++j) o = fmaf(w[j], y[(size_t)j * H + c], o);
    o = fmaf(g, y[(size_t)k * H + c], o);
    out[c] = o;
    ss = fmaf(o, o, ss);
  }
  if (!out_norm) return;
  ss = block_sum(ss, red);
  const float xs = 1.f / sqrtf(ss / (float)H + eps);
  for (int c = threadIdx.x; c < H; c += blockDim.x) out_norm[c] = out[c] * xs;
}

// strided record copy, 16 bytes per thread step
__global__ void pack_kernel(const uint4* __restrict__ src, int64_t src_stride16, uint4* dst,
                            int64_t dst_stride16, int64_t rec16, int n) {
  const int64_t total = rec16 * n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t s = i / rec16, o = i - s * rec16;
    dst[s * dst_stride16 + o] = src[s * src_stride16 + o];
  }
}

// column-blocked router copy: dst[c][e][0..15] = src[e][16 c .. 16 c + 15], one 64-byte
// segment per thread
__global__ void pack_router_kernel(const float4* __restrict__ src, int n_experts, int hidden,
                                   float4* __restrict__ dst) {
  const int64_t nseg = (int64_t)n_experts * (hidden / 16);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nseg;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = i / n_experts, e = i - c * n_experts;  // dst order: block c, expert e
    const float4* s = src + (e * hidden + 16 * c) / 4;
    float4* d = dst + 4 * i;
#pragma unroll
    for (int k = 0; k < 4; ++k) d[k] = s[k];
  }
}

// ------------------------------------------------------------------------------------------
// launch helpers (template dispatch over the supported shapes)
// ------------------------------------------------------------------------------------------
inline moe_status last_error() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP; }

template <int BITS, bool SHARED, int NTOK>
void launch_k1_bs(const K1Args& a, int H, dim3 grid, hipStream_t s) {
  switch (H) {
    case 1024:
      hipLaunchKernelGGL((k1_kernel<BITS, 1024, SHARED, NTOK>), grid, dim3(kBlock), 0, s, a);
      break;
    case 2048:
      hipLaunchKernelGGL((k1_kernel<BITS, 2048, SHARED, NTOK>), grid, dim3(kBlock), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((k1_kernel<BITS, 4096, SHARED, NTOK>), grid, dim3(kBlock), 0, s, a);
      break;
  }
}
// tokens staged together by a K1 block running the shared expert over several tokens
constexpr int kK1Group = 4;
constexpr int kRouteTokens = 3;  // tokens from which run_layer routes in a launch of its own
// router rows for a.T tokens (one grid row per token); with a shared expert also its gate/up
// rows, each block running its rows over the tokens
inline int k1_dig_tokens_h(int H) {
  return H == 1024 ? k1_dig_tokens<1024>() : H == 2048 ? k1_dig_tokens<2048>() : k1_dig_tokens<4096>();
}

void launch_k1(const K1Args& a, int bits, int H, hipStream_t s) {
  const int rb = (a.E + 1) / 2;
  const int sb = a.shared ? a.I / 4 : 0;
  const dim3 grid((rb > sb ? rb : sb) + (a.sg_ws ? 1 : 0) + a.dig_blocks, a.shared ? 1 : a.T);
  if (!a.shared)
    launch_k1_bs<4, false, 1>(a, H, grid, s);
  else if (bits == 4)
    a.T == 1 ? launch_k1_bs<4, true, 1>(a, H, grid, s)
             : launch_k1_bs<4, true, kK1Group>(a, H, grid, s);
  else
    a.T == 1 ? launch_k1_bs<2, true, 1>(a, H, grid, s)
             : launch_k1_bs<2, true, kK1Group>(a, H, grid, s);
}

// waves per K2 block: 8 for four to seven slots (one token); fewer below, so that the grid
// keeps filling the chip, and 4 from eight slots up (several tokens), where three blocks per
// CU overlap one block's top-k and load latency with the others' streaming
inline int k2_waves(int n) { return n >= 8 ? 4 : n >= 4 ? 8 : n >= 2 ? 4 : 2; }

template <int BITS, int H, int WAVES>
void launch_k2_w(const K2Args& a, hipStream_t s) {
  const dim3 grid(a.n * (a.I / k2_rows_per_block<BITS, H, WAVES>()));
  if (a.xdig)
    hipLaunchKernelGGL((k2_kernel<BITS, H, WAVES, true>), grid, dim3(64 * WAVES), 0, s, a);
  else
    hipLaunchKernelGGL((k2_kernel<BITS, H, WAVES, false>), grid, dim3(64 * WAVES), 0, s, a);
}
template <int BITS, int H>
void launch_k2_h(const K2Args& a, hipStream_t s) {
  switch (k2_waves(a.n)) {
    case 8: launch_k2_w<BITS, H, 8>(a, s); break;
    case 4: launch_k2_w<BITS, H, 4>(a, s); break;
    default: launch_k2_w<BITS, H, 2>(a, s); break;
  }
}
template <int BITS>
void launch_k2_b(const K2Args& a, int H, hipStream_t s) {
  switch (H) {
    case 1024: launch_k2_h<BITS, 1024>(a, s); break;
    case 2048: launch_k2_h<BITS, 2048>(a, s); break;
    default: launch_k2_h<BITS, 4096>(a, s); break;
  }
}
void launch_k2(const K2Args& a, int bits, int H, hipStream_t s) {
  if (bits == 4) launch_k2_b<4>(a, H, s); else launch_k2_b<2>(a, H, s);
}

// waves per slot in a K3 block: 8 for one slot down to 1 from five slots up, and never more
// than the slot has row blocks
template <int BITS, int I, int KW>
void launch_k3_kw(const K3Args& a, int T, hipStream_t s) {
  if constexpr (k3_row_blocks<BITS, I>() % KW == 0)
    hipLaunchKernelGGL((k3_kernel<BITS, I, KW>), dim3(a.H / kDownRows, T), dim3(64 * a.n * KW),
                       0, s, a);
}
template <int BITS, int I>
void launch_k3_i(const K3Args& a, int T, hipStream_t s) {
  int kw = a.n >= 5 ? 1 : a.n >= 3 ? 2 : a.n == 2 ? 4 : 8;
  while (kw > 1 && k3_row_blocks<BITS, I>() % kw) kw >>= 1;
  switch (kw) {
    case 8: launch_k3_kw<BITS, I, 8>(a, T, s); break;
    case 4: launch_k3_kw<BITS, I, 4>(a, T, s); break;
    case 2: launch_k3_kw<BITS, I, 2>(a, T, s); break;
    default: launch_k3_kw<BITS, I, 1>(a, T, s); break;
  }
}
template <int BITS>
void launch_k3_b(const K3Args& a, int I, int T, hipStream_t s) {
  switch (I) {
    case 256: launch_k3_i<BITS, 256>(a, T, s); break;
    case 512: launch_k3_i<BITS, 512>(a, T, s); break;
    case 1024: launch_k3_i<BITS, 1024>(a, T, s); break;
    default: launch_k3_i<BITS, 2048>(a, T, s); break;
  }
}
void launch_k3(const K3Args& a, int bits, int I, int T, hipStream_t s) {
  if (bits == 4) launch_k3_b<4>(a, I, T, s); else launch_k3_b<2>(a, I, T, s);
}

template <int BITS>
void launch_qgemv_b(const uint8_t* rec, int R, int C, const float* x, float* y, hipStream_t s) {
  auto grid_for = [&](int rows_per_wave) {
    const int nrb = (R + rows_per_wave - 1) / rows_per_wave;
    const int waves = (nrb + 3) / 4;
    return dim3((waves + 3) / 4);
  };
  switch (C) {
    case 256: hipLaunchKernelGGL((qgemv_kernel<BITS, 256>), grid_for(Geo<BITS, 256>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    case 512: hipLaunchKernelGGL((qgemv_kernel<BITS, 512>), grid_for(Geo<BITS, 512>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    case 1024: hipLaunchKernelGGL((qgemv_kernel<BITS, 1024>), grid_for(Geo<BITS, 1024>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    case 2048: hipLaunchKernelGGL((qgemv_kernel<BITS, 2048>), grid_for(Geo<BITS, 2048>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    case 4096: hipLaunchKernelGGL((qgemv_kernel<BITS, 4096>), grid_for(Geo<BITS, 4096>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    default: hipLaunchKernelGGL((qgemv_kernel<BITS, 8192>), grid_for(Geo<BITS, 8192>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
  }
}

// One decode layer for T tokens on a prepared workspace: K1 -> K2 -> K3.
struct LayerCall {
  const moe_layer* L;
  const float* x;      // [T][H] residual (layer input)
  int T;
  int norm;            // router and experts see RMSNorm(x)
  float eps;
  float* out;          // [T][H]
  int32_t* ids_out;    // optional [T][k (+1)]
  float* weights_out;  // optional [T][k]
  float* sg_out;       // optional [T]
  int32_t* ids_trace;  // optional [T][k]
};

moe_status run_layer(const LayerCall& c, uint8_t* ws, const LayerWs& lw, hipStream_t s) {
  const moe_layer* L = c.L;
  const moe_experts& X = L->experts;
  const int H = X.hidden, I = X.inter, E = L->n_experts, k = L->top_k;
  const bool has_shared = L->shared_slot >= 0;
  const int hpt = k + (has_shared ? 1 : 0);  // h rows (and ids) per token
  const uint8_t* base = reinterpret_cast<const uint8_t*>(X.base);
  float* logits = reinterpret_cast<float*>(ws + lw.logits);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + lw.ids);
  float* weights = reinterpret_cast<float*>(ws + lw.weights);
  float* sg = reinterpret_cast<float*>(ws + lw.sg);
  float* h = reinterpret_cast<float*>(ws + lw.h);

  K1Args a1{};
  a1.x = c.x;
  a1.T = c.T;
  a1.norm = c.norm;
  a1.eps = c.eps;
  a1.w_router = L->w_router;
  a1.E = E;
  a1.logits = logits;
  a1.shared = has_shared ? base + (size_t)L->shared_slot * X.slot_bytes : nullptr;
  a1.I = I;
  a1.h_shared = h + (size_t)k * I;
  a1.h_stride = (int64_t)hpt * I;
  a1.w_sg = L->w_sg;
  a1.sg_ws = sg;
  a1.sg_out = c.sg_out;
  // K1's trailing blocks build the digit planes of the inputs for K2's products
  uint4* xdig = reinterpret_cast<uint4*>(ws + lw.xdig);
  float* xscale = reinterpret_cast<float*>(ws + lw.xscale);
  a1.xdig = xdig;
  a1.xscale = xscale;
  a1.dig_even_odd = X.bits == 2;
  a1.dig_blocks = (c.T + k1_dig_tokens_h(H) - 1) / k1_dig_tokens_h(H);
  launch_k1(a1, X.bits, H, s);

  K2Args a2{};
  a2.x = c.x;
  a2.norm = c.norm;
  a2.eps = c.eps;
  a2.logits = logits;
  a2.E = E;
  a2.k = k;
  a2.n = c.T * k;
  a2.base = base;
  a2.slot_bytes = X.slot_bytes;
  a2.n_slots_total = X.n_slots;
  a2.I = I;
  a2.h = h;
  a2.h_per_token = hpt;
  a2.ids_ws = ids;
  a2.w_ws = weights;
  a2.shared_slot = L->shared_slot;
  a2.ids_out = c.ids_out;
  a2.w_out = c.weights_out;
  a2.ids_trace = c.ids_trace;
  a2.dev_err = X.dev_err;
  a2.xdig = xdig;
  a2.xscale = xscale;
  // from kRouteTokens tokens on, one routing launch instead of a top-k in every K2 block
  a2.routed = c.T >= kRouteTokens;
  if (a2.routed) hipLaunchKernelGGL(route_kernel, dim3(c.T), dim3(64), 0, s, a2);
  launch_k2(a2, X.bits, H, s);

  K3Args a3{};
  a3.base = base;
  a3.slot_bytes = X.slot_bytes;
  a3.n_slots_total = X.n_slots;
  a3.ids = ids;
  a3.n = hpt;
  a3.h = h;
  a3.H = H;
  a3.y = nullptr;
  a3.residual = c.x;
  a3.route_w = weights;
  a3.n_routed = k;
  a3.sg = sg;
  a3.out = c.out;
  a3.dev_err = X.dev_err;
  launch_k3(a3, X.bits, I, c.T, s);
  return last_error();
}

// ------------------------------------------------------------------------------------------
// Scratch for moe_decode_stack_static: a file-scope device array instead of a caller workspace.
// Each device holds its own copy; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device (the array's name in host code is a
// host-side stand-in, not a device address).
// ------------------------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(2) << 20;
constexpr int kMaxDevices = 64;

__global__ void zero_fill_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
struct DeviceScratch {
  std::once_flag once;
  uint8_t* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// This device's scratch, resolved and zero-filled (on `stream`, ahead of the caller's kernels)
// by the first call on the device; nullptr if that failed.
uint8_t* device_scratch(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&] {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.err != hipSuccess || !p) {
      if (d.err == hipSuccess) d.err = hipErrorInvalidSymbol;
      return;
    }
    hipLaunchKernelGGL(zero_fill_kernel, dim3(256), dim3(256), 0, stream,
                       reinterpret_cast<uint4*>(p), kStaticScratchBytes / 16);
    d.err = hipGetLastError();
    if (d.err == hipSuccess) d.ptr = reinterpret_cast<uint8_t*>(p);
  });
  return d.err == hipSuccess ? d.ptr : nullptr;
}
}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_NULL: return "required pointer is NULL";
    case MOE_E_SHAPE: return "unsupported or inconsistent shape";
    case MOE_E_ALIGN: return "pointer or stride not 16-byte aligned";
    case MOE_E_BITS: return "bits must be 4 or 2";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    case MOE_E_HIP: return "HIP launch error";
  }
  return "unknown status";
}

const char* moe_version(void) { return "libmoe 0.2 gfx950"; }

size_t moe_router_workspace_bytes(int T, int E) {
  if (T < 1 || E < 1) return 0;
  return align_up((size_t)T * E * sizeof(float));
}

moe_status moe_router_topk(const float* x, int T, const float* w_router, const float* w_sg,
                           int H, int E, int k, int32_t* ids, int ld_ids, float* weights,
                           float* shared_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!x || !w_router || !ids || !weights) return MOE_E_NULL;
  if (T < 1 || T > 65535 || !hidden_ok(H) || E < 1 || E > 1024 || k < 1 || k > kMaxTopK ||
      k > E || ld_ids < k)
    return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(w_router) || (w_sg && !aligned16(w_sg))) return MOE_E_ALIGN;
  if (!ws || ws_bytes < moe_router_workspace_bytes(T, E)) return MOE_E_WORKSPACE;
  float* logits = reinterpret_cast<float*>(ws);
  K1Args a1{};
  a1.x = x;
  a1.T = T;
  a1.norm = 0;
  a1.w_router = w_router;
  a1.E = E;
  a1.logits = logits;
  a1.shared = nullptr;
  a1.I = 4;
  launch_k1(a1, 4, H, stream);
  hipLaunchKernelGGL(topk_kernel, dim3(T), dim3(64), 0, stream, logits, E, k, x, w_sg, H, ids,
                     ld_ids, weights, shared_gate);
  return last_error();
}

static moe_status expert_ffn(int bits, const moe_experts* w, const float* x, const int32_t* ids,
                             int n, float* y, float* h, hipStream_t stream) {
  moe_status st = check_experts(w);
  if (st != MOE_OK) return st;
  if (w->bits != bits) return MOE_E_BITS;
  if (!x || !ids || !y || !h) return MOE_E_NULL;
  if (n < 1 || n > 8) return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(h)) return MOE_E_ALIGN;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(w->base);
  K2Args a2{};
  a2.x = x;
  a2.norm = 0;
  a2.logits = nullptr;
  a2.ids_in = ids;
  a2.n = n;
  a2.base = base;
  a2.slot_bytes = w->slot_bytes;
  a2.n_slots_total = w->n_slots;
  a2.I = w->inter;
  a2.h = h;
  a2.shared_slot = -1;
  a2.dev_err = w->dev_err;
  launch_k2(a2, bits, w->hidden, stream);
  K3Args a3{};
  a3.base = base;
  a3.slot_bytes = w->slot_bytes;
  a3.n_slots_total = w->n_slots;
  a3.ids = ids;
  a3.n = n;
  a3.h = h;
  a3.H = w->hidden;
  a3.y = y;
  a3.dev_err = w->dev_err;
  launch_k3(a3, bits, w->inter, 1, stream);
  return last_error();
}

moe_status moe_expert_ffn_q4(const moe_experts* w, const float* x, const int32_t* ids, int n,
                             float* y, float* h, hipStream_t stream) {
  return expert_ffn(4, w, x, ids, n, y, h, stream);
}

moe_status moe_expert_ffn_q2(const moe_experts* w, const float* x, const int32_t* ids, int n,
                             float* y, float* h, hipStream_t stream) {
  return expert_ffn(2, w, x, ids, n, y, h, stream);
}

moe_status moe_combine(const float* residual, const float* y, const float* weights, int k,
                       const float* shared_gate, float* out, float* out_norm, float eps, int H,
                       hipStream_t stream) {
  if (!residual || !y || !weights || !out) return MOE_E_NULL;
  if (k < 0 || k > kMaxTopK || H < 1) return MOE_E_SHAPE;
  hipLaunchKernelGGL(combine_kernel, dim3(1), dim3(1024), 0, stream, residual, y, weights, k,
                     shared_gate, out, out_norm, eps, H);
  return last_error();
}

size_t moe_layer_workspace_bytes(const moe_layer* layer) {
  if (check_layer(layer) != MOE_OK) return 0;
  return LayerWs::make(layer->experts.hidden, layer->experts.inter, layer->n_experts,
                       layer->top_k, false).total;
}

moe_status moe_layer_decode(const moe_layer* layer, const float* x, int norm_input, float eps,
                            float* out, int32_t* ids_out, float* weights_out, float* sg_out,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !out) return MOE_E_NULL;
  if (!aligned16(x) || !aligned16(out)) return MOE_E_ALIGN;
  if (x == out) return MOE_E_SHAPE;
  const LayerWs lw = LayerWs::make(layer->experts.hidden, layer->experts.inter,
                                   layer->n_experts, layer->top_k, false);
  if (!ws || ws_bytes < lw.total) return MOE_E_WORKSPACE;
  LayerCall c{};
  c.L = layer;
  c.x = x;
  c.T = 1;
  c.norm = norm_input ? 1 : 0;
  c.eps = eps;
  c.out = out;
  c.ids_out = ids_out;
  c.weights_out = weights_out;
  c.sg_out = sg_out;
  return run_layer(c, reinterpret_cast<uint8_t*>(ws), lw, stream);
}

size_t moe_stack_workspace_bytes(const moe_layer* layers, int n_layers) {
  if (!layers || n_layers < 1 || check_layer(&layers[0]) != MOE_OK) return 0;
  return LayerWs::make(layers[0].experts.hidden, layers[0].experts.inter, layers[0].n_experts,
                       layers[0].top_k, true).total +
         align_up(PersistWs::bytes());
}

moe_status moe_decode_stack(const moe_layer* layers, int n_layers, const float* x_in,
                            float* x_out, float* xn_out, float eps, int32_t* ids_trace,
                            int flags, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!layers || !x_in || !x_out) return MOE_E_NULL;
  if (n_layers < 1) return MOE_E_SHAPE;
  const int mode = flags & ~MOE_STACK_PLAIN_LAUNCH;
  if (mode != MOE_STACK_AUTO && mode != MOE_STACK_KERNELS && mode != MOE_STACK_PERSISTENT)
    return MOE_E_SHAPE;
  const bool plain = (flags & MOE_STACK_PLAIN_LAUNCH) != 0;
  for (int l = 0; l < n_layers; ++l) {
    moe_status st = check_layer(&layers[l]);
    if (st != MOE_OK) return st;
    const moe_layer& a = layers[l];
    const moe_layer& b = layers[0];
    if (a.experts.hidden != b.experts.hidden || a.experts.inter != b.experts.inter ||
        a.experts.bits != b.experts.bits || a.n_experts != b.n_experts || a.top_k != b.top_k ||
        (a.shared_slot >= 0) != (b.shared_slot >= 0))
      return MOE_E_SHAPE;
  }
  if (!aligned16(x_in) || !aligned16(x_out) || (xn_out && !aligned16(xn_out)))
    return MOE_E_ALIGN;
  if (x_in == x_out || xn_out == x_out) return MOE_E_SHAPE;
  const int H = layers[0].experts.hidden;
  const LayerWs lw = LayerWs::make(H, layers[0].experts.inter, layers[0].n_experts,
                                   layers[0].top_k, true);
  if (!ws || ws_bytes < lw.total) return MOE_E_WORKSPACE;
  if (ws_bytes < lw.total + align_up(PersistWs::bytes())) return MOE_E_WORKSPACE;
  uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
  float* xbuf = reinterpret_cast<float*>(w8 + lw.xbuf);
  const int k = layers[0].top_k;
  const bool persist = mode != MOE_STACK_KERNELS && persist_shape_ok(layers, n_layers) &&
                       persist_device_ok();
  if (mode == MOE_STACK_PERSISTENT && !persist) return MOE_E_SHAPE;
  if (persist) {
    // chunks of at most kPersistMaxLayers layers; raw x passes between chunks through xbuf
    for (int l0 = 0, c = 0; l0 < n_layers; l0 += kPersistMaxLayers, ++c) {
      const int nl = n_layers - l0 < kPersistMaxLayers ? n_layers - l0 : kPersistMaxLayers;
      const bool last = l0 + nl == n_layers;
      const float* xi = l0 == 0 ? x_in : xbuf + (size_t)((c - 1) & 1) * H;
      float* xo = last ? x_out : xbuf + (size_t)(c & 1) * H;
      moe_status st = persist_launch(layers + l0, nl, xi, xo, last ? xn_out : nullptr, eps,
                                     ids_trace ? ids_trace + (size_t)l0 * k : nullptr,
                                     w8 + lw.total, plain, stream);
      if (st != MOE_OK) return st;
    }
    return last_error();
  }
  for (int l = 0; l < n_layers; ++l) {
    LayerCall c{};
    c.L = &layers[l];
    c.T = 1;
    c.x = l == 0 ? x_in : xbuf + (size_t)((l - 1) & 1) * H;
    c.out = l == n_layers - 1 ? x_out : xbuf + (size_t)(l & 1) * H;
    c.norm = 1;
    c.eps = eps;
    c.ids_trace = ids_trace ? ids_trace + (size_t)l * k : nullptr;
    moe_status st = run_layer(c, w8, lw, stream);
    if (st != MOE_OK) return st;
  }
  if (xn_out) hipLaunchKernelGGL(rmsnorm_kernel, dim3(1), dim3(1024), 0, stream, x_out, H, eps, xn_out);
  return last_error();
}

size_t moe_layer_batch_workspace_bytes(const moe_layer* layer, int T) {
  if (check_layer(layer) != MOE_OK || T < 1 || T > kMaxBatch) return 0;
  return LayerWs::make(layer->experts.hidden, layer->experts.inter, layer->n_experts,
                       layer->top_k, false, T).total;
}

moe_status moe_layer_decode_batch(const moe_layer* layer, const float* x, int T, int norm_input,
                                  float eps, float* out, int32_t* ids_out, float* weights_out,
                                  float* sg_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !out) return MOE_E_NULL;
  if (T < 1 || T > kMaxBatch) return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(out)) return MOE_E_ALIGN;
  const size_t xb = (size_t)T * layer->experts.hidden * sizeof(float);
  const uint8_t *xp = reinterpret_cast<const uint8_t*>(x), *op = reinterpret_cast<const uint8_t*>(out);
  if (xp < op + xb && op < xp + xb) return MOE_E_SHAPE;  // out overlaps x
  const LayerWs lw = LayerWs::make(layer->experts.hidden, layer->experts.inter,
                                   layer->n_experts, layer->top_k, false, T);
  if (!ws || ws_bytes < lw.total) return MOE_E_WORKSPACE;
  LayerCall c{};
  c.L = layer;
  c.x = x;
  c.T = T;
  c.norm = norm_input ? 1 : 0;
  c.eps = eps;
  c.out = out;
  c.ids_out = ids_out;
  c.weights_out = weights_out;
  c.sg_out = sg_out;
  return run_layer(c, reinterpret_cast<uint8_t*>(ws), lw, stream);
}

size_t moe_stack_batch_workspace_bytes(const moe_layer* layers, int n_layers, int T) {
  if (!layers || n_layers < 1 || T < 1 || T > kMaxBatch || check_layer(&layers[0]) != MOE_OK)
    return 0;
  return LayerWs::make(layers[0].experts.hidden, layers[0].experts.inter, layers[0].n_experts,
                       layers[0].top_k, true, T).total;
}

moe_status moe_decode_stack_batch(const moe_layer* layers, int n_layers, const float* x_in,
                                  int T, float* x_out, float* xn_out, float eps,
                                  int32_t* ids_trace, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (!layers || !x_in || !x_out) return MOE_E_NULL;
  if (n_layers < 1 || T < 1 || T > kMaxBatch) return MOE_E_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    moe_status st = check_layer(&layers[l]);
    if (st != MOE_OK) return st;
    const moe_layer& a = layers[l];
    const moe_layer& b = layers[0];
    if (a.experts.hidden != b.experts.hidden || a.experts.inter != b.experts.inter ||
        a.experts.bits != b.experts.bits || a.n_experts != b.n_experts || a.top_k != b.top_k ||
        (a.shared_slot >= 0) != (b.shared_slot >= 0))
      return MOE_E_SHAPE;
  }
  if (!aligned16(x_in) || !aligned16(x_out) || (xn_out && !aligned16(xn_out)))
    return MOE_E_ALIGN;
  const int H = layers[0].experts.hidden, k = layers[0].top_k;
  const size_t xb = (size_t)T * H * sizeof(float);
  auto overlap = [xb](const void* p, const void* q) {
    const uint8_t *a = reinterpret_cast<const uint8_t*>(p), *b = reinterpret_cast<const uint8_t*>(q);
    return a < b + xb && b < a + xb;
  };
  if (overlap(x_in, x_out) || (xn_out && overlap(xn_out, x_out))) return MOE_E_SHAPE;
  const LayerWs lw = LayerWs::make(H, layers[0].experts.inter, layers[0].n_experts, k, true, T);
  if (!ws || ws_bytes < lw.total) return MOE_E_WORKSPACE;
  uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
  float* xbuf = reinterpret_cast<float*>(w8 + lw.xbuf);
  for (int l = 0; l < n_layers; ++l) {
    LayerCall c{};
    c.L = &layers[l];
    c.T = T;
    c.x = l == 0 ? x_in : xbuf + (size_t)((l - 1) & 1) * T * H;
    c.out = l == n_layers - 1 ? x_out : xbuf + (size_t)(l & 1) * T * H;
    c.norm = 1;
    c.eps = eps;
    c.ids_trace = ids_trace ? ids_trace + (size_t)l * T * k : nullptr;
    moe_status st = run_layer(c, w8, lw, stream);
    if (st != MOE_OK) return st;
  }
  if (xn_out)
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(1024), 0, stream, x_out, H, eps, xn_out);
  return last_error();
}

moe_status moe_decode_stack_static(const moe_layer* layers, int n_layers, const float* x_in,
                                   float* x_out, float* xn_out, float eps, int32_t* ids_trace,
                                   int flags, hipStream_t stream) {
  if (!layers) return MOE_E_NULL;
  const size_t need = moe_stack_workspace_bytes(layers, n_layers);
  if (need == 0) return moe_decode_stack(layers, n_layers, x_in, x_out, xn_out, eps, ids_trace,
                                         flags, nullptr, 0, stream);  // its validation status
  if (need > kStaticScratchBytes) return MOE_E_WORKSPACE;
  uint8_t* ws = device_scratch(stream);
  if (!ws) return MOE_E_HIP;
  return moe_decode_stack(layers, n_layers, x_in, x_out, xn_out, eps, ids_trace, flags, ws,
                          kStaticScratchBytes, stream);
}

moe_status moe_qgemv(const moe_qmatrix* m, const float* x, float* y, hipStream_t stream) {
  if (!m || !m->rec || !x || !y) return MOE_E_NULL;
  if (m->bits != 4 && m->bits != 2) return MOE_E_BITS;
  if (m->group != 64 || m->rows < 1 ||
      !(m->cols == 256 || m->cols == 512 || m->cols == 1024 || m->cols == 2048 ||
        m->cols == 4096 || m->cols == 8192))
    return MOE_E_SHAPE;
  if (!aligned16(m->rec) || !aligned16(x)) return MOE_E_ALIGN;
  const uint8_t* rec = reinterpret_cast<const uint8_t*>(m->rec);
  if (m->bits == 4)
    launch_qgemv_b<4>(rec, m->rows, m->cols, x, y, stream);
  else
    launch_qgemv_b<2>(rec, m->rows, m->cols, x, y, stream);
  return last_error();
}

moe_status moe_rmsnorm(const float* x, int T, int H, float eps, float* out,
                       hipStream_t stream) {
  if (!x || !out) return MOE_E_NULL;
  if (T < 1 || H < 1) return MOE_E_SHAPE;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(1024), 0, stream, x, H, eps, out);
  return last_error();
}

moe_status moe_pack(const void* canonical, int n, int slot0, const moe_experts* dst,
                    hipStream_t stream) {
  moe_status st = check_experts(dst);
  if (st != MOE_OK) return st;
  if (!canonical) return MOE_E_NULL;
  if (n < 1 || slot0 < 0 || slot0 + n > dst->n_slots) return MOE_E_SHAPE;
  if (!aligned16(canonical)) return MOE_E_ALIGN;
  const int64_t rec = expert_bytes(dst->bits, dst->hidden, dst->inter);
  if (rec % 16) return MOE_E_ALIGN;
  uint8_t* base = reinterpret_cast<uint8_t*>(const_cast<void*>(dst->base)) +
                  (size_t)slot0 * dst->slot_bytes;
  hipLaunchKernelGGL(pack_kernel, dim3(1024), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(canonical), rec / 16,
                     reinterpret_cast<uint4*>(base), dst->slot_bytes / 16, rec / 16, n);
  return last_error();
}

moe_status moe_pack_router(const float* w_router, int n_experts, int hidden, float* dst,
                           hipStream_t stream) {
  if (!w_router || !dst) return MOE_E_NULL;
  if (n_experts < 1 || hidden < 16 || hidden % 16) return MOE_E_SHAPE;
  if (!aligned16(w_router) || !aligned16(dst)) return MOE_E_ALIGN;
  hipLaunchKernelGGL(pack_router_kernel, dim3(1024), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(w_router), n_experts, hidden,
                     reinterpret_cast<float4*>(dst));
  return last_error();
}

}  // extern "C"
