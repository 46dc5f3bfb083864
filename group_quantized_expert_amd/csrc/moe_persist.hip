// moe_persist.hip -- one launch per token: the whole q4 MoE layer stack decoded by a
// persistent grid of one workgroup per compute unit.
//
// Why: a decode layer moves ~44 MB but is a chain of three grid-wide dependencies (the layer
// input feeds the router, the router's top-k picks the expert rows every workgroup loads, the
// SwiGLU activations h of every expert feed every down row).  As separate kernels each link
// costs a launch plus a cold start of dependent loads.  Here the links are in-kernel
// exchanges, and every weight load that does not depend on the current routing (the next
// layer's router rows and shared-expert gate/up rows) is issued into registers while the
// routed experts stream, so HBM stays busy across the dependency waits.
//
// Shape (the Qwen3.5-397B-A17B MoE block: jeongsk-2ndbrain.pages.dev Flash-MoE wiki, "Target
// model"; a2a-mcp.org "What is Flash-MoE", MoE section): H = 4096, I = 1024, E = 512 routed
// experts, top-4 plus one shared expert, q4 codes, group 64, bf16 scale and bias.  Other shapes
// and q2 use the kernel-per-step path in moe_decode.hip.
//
// Grid: 256 workgroups, one per CU (cooperative launch), 12 waves each:
//   waves 0-7  (compute)  weight loads into registers and all dot products;
//   waves 8-11 (exchange) publish this workgroup's results and gather everyone's.
// The split keeps the exchange polls off the compute waves' in-order load counter: a poll
// in a compute wave would first wait for every weight load issued before it.
//
// Exchange (all-gather of tagged words).  A word is (fp32 value | tag << 32), written with
// one 64-bit store, so a reader checks freshness per word and needs no flag or fence.  Tags
// are epoch + layer + 1 and never repeat within a workspace.  Two levels: workgroup (x, j)
// (x = XCD, j = 0..31) fetches slice j of the global words with device-coherent loads and
// stores it into its XCD's staging copy; every workgroup then polls its own XCD's copy, which
// its shared L2 serves.  Each global word is therefore polled by 8 readers, not 256.  Every
// poll is bounded in time; on expiry the workgroup stops waiting for the rest of the launch
// and the error is reported through the layer's dev_err word.
//
// Per-layer buffer reuse is safe without double buffering: a workgroup rewrites an exchange
// buffer for layer L+1 only after a later exchange of layer L has completed, which every
// workgroup joins only after it finished reading that buffer for layer L.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "moe.h"
#include "moe_device.h"
#include "moe_host.h"
#include "moe_persist.h"

namespace moe {
namespace {

constexpr int kPB = 256;                 // workgroups
constexpr int kPX = 8;                   // XCDs
constexpr int kPJ = kPB / kPX;           // workgroups per XCD
constexpr int kPH = 4096, kPI = 1024, kPE = 512, kPK = 4;
constexpr int kPS = kPK + 1;             // expert slots per layer (routed + shared)
constexpr int kCW = 8, kXW = 4;          // compute / exchange waves
constexpr int kPT = (kCW + kXW) * kWave; // 768 threads
constexpr int kXT = kXW * kWave;         // exchange threads
constexpr uint64_t kSpinTicks = 20000000;  // 200 ms of the 100 MHz real-time counter

// record geometry (q4, group 64)
constexpr size_t kGuCodes = (size_t)kPI * kPH / 2;               // 2 MiB
constexpr size_t kGuMeta = (size_t)kPI * (kPH / kGroup) * 2;     // 128 KiB (scale or bias)
constexpr size_t kGuRec = kGuCodes + 2 * kGuMeta;                // 2,359,296
constexpr size_t kDnCodes = (size_t)kPH * kPI / 2;
constexpr size_t kDnMeta = (size_t)kPH * (kPI / kGroup) * 2;
constexpr size_t kDnOff = 2 * kGuRec;                            // down record in a slot

// exchange sizes (words)
constexpr int kNOut = kPH, kNLogit = kPE, kNH = kPS * kPI;

struct PLayer {
  const uint8_t* base;
  const float* w_router;
  const float* w_sg;
  int64_t slot_bytes;
  int32_t n_slots;
  int32_t shared_slot;
};

struct PArgs {
  PLayer layer[kPersistMaxLayers];
  int n_layers;
  float eps;
  const float* x_in;
  float* x_out;
  float* xn_out;
  int32_t* ids_trace;
  uint8_t* xw;       // exchange area (PersistWs layout)
  int32_t* dev_err;
};

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---- exchange memory access (buffer instructions with explicit cache policy) ----
// aux 16 = sc1: device-coherent (reaches memory; a load does not hit a stale L1/L2 copy).
// aux 0 = default: stores land in the XCD's L2, which the XCD's readers share.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
}
template <int AUX>
__device__ __forceinline__ u32x4 xld(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ void xst2(__amdgpu_buffer_rsrc_t r, int byte_off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, AUX);
}
__device__ __forceinline__ void xst1(__amdgpu_buffer_rsrc_t r, int word, float v, uint32_t tag) {
  u32x2 w;
  w.x = __float_as_uint(v);
  w.y = tag;
  __builtin_amdgcn_raw_buffer_store_b64(w, r, word * 8, 0, 16);
}

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Barrier of all 12 waves.  Waits for this wave's LDS operations, not for its outstanding
// global loads (those are the prefetches that must stay in flight).
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) int lds_int;

struct XCtx {
  int b, j, t;          // workgroup, its slot within the XCD, exchange thread 0..255
  uint32_t xcc;         // hardware XCD id of this workgroup
  lds_int* abort;       // LDS flag: stop waiting (set on timeout or bad placement)
  int32_t* err;         // exchange-area error word
  int32_t* dev_err;
};

__device__ __forceinline__ void fail(const XCtx& c, int code) {
  *(volatile lds_int*)c.abort = 1;
  atomicOr(c.err, code);
  if (c.dev_err) atomicOr(c.dev_err, code);
}

// Poll K pairs (16-byte units of two tagged words) p = t + NTH i of buffer r until both tags
// of each equal tag; returns the values (2 per pair).
template <int K, int NPAIR, int NTH, int AUX>
__device__ __forceinline__ void poll_pairs(const XCtx& c, int t, __amdgpu_buffer_rsrc_t r,
                                           uint32_t tag, float (&v)[2 * K]) {
  const uint64_t t0 = now_ticks();
  while (true) {
    u32x4 w[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int p = t + NTH * i;
      w[i] = xld<AUX>(r, (p < NPAIR ? p : 0) * 16);
    }
    bool ok = true;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int p = t + NTH * i;
      if (p < NPAIR) ok = ok && w[i].y == tag && w[i].w == tag;
    }
    if (ok) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        v[2 * i] = __uint_as_float(w[i].x);
        v[2 * i + 1] = __uint_as_float(w[i].z);
      }
      return;
    }
    if (*(volatile lds_int*)c.abort) break;
    if (now_ticks() - t0 > kSpinTicks) {
      fail(c, kPersistErrTimeout);
      break;
    }
  }
#pragma unroll
  for (int i = 0; i < 2 * K; ++i) v[i] = 0.f;
}

// All-gather of N tagged words by NTH exchange threads (t = 0 .. NTH-1): fetch slice j of the
// global buffer into this XCD's staging copy, then poll the staging copy.  Thread t receives
// words 2p, 2p+1 for p = t + NTH i.
template <int N, int NTH>
__device__ __forceinline__ void gather(const XCtx& c, int t, uint64_t* g, uint64_t* stage,
                                       uint32_t tag, float (&v)[2 * (N / 2 / NTH)]) {
  constexpr int kFetch = N / 64;            // pairs fetched by each workgroup of an XCD
  constexpr int kLocal = N / 2 / NTH;       // pairs polled per thread
  static_assert(N % (2 * NTH) == 0 && kFetch <= NTH, "");
  const auto rg = rsrc(g);
  const auto rl = rsrc(stage + (size_t)(c.xcc & (kPX - 1)) * N);
  if (t < kFetch && !*(volatile lds_int*)c.abort) {
    // two polls in flight, so the words are seen within about one round trip of landing
    const int p = c.j * kFetch + t;
    const uint64_t t0 = now_ticks();
    u32x4 w0 = xld<16>(rg, p * 16);
    while (true) {
      const u32x4 w1 = xld<16>(rg, p * 16);
      if (w0.y == tag && w0.w == tag) {
        xst2<0>(rl, p * 16, w0);
        break;
      }
      w0 = xld<16>(rg, p * 16);
      if (w1.y == tag && w1.w == tag) {
        xst2<0>(rl, p * 16, w1);
        break;
      }
      if (*(volatile lds_int*)c.abort) break;
      if (now_ticks() - t0 > kSpinTicks) {
        fail(c, kPersistErrTimeout);
        break;
      }
    }
  }
  if (*(volatile lds_int*)c.abort) {
#pragma unroll
    for (int i = 0; i < 2 * kLocal; ++i) v[i] = 0.f;
    return;
  }
  poll_pairs<kLocal, N / 2, NTH, 16>(c, t, rl, tag, v);
}

constexpr int kDppRowHalfMirror = 0x141;  // row_half_mirror: lane i of each 8 <- lane 7 - i

// ---- routing: top-k of the 512 logits in two steps ----
// A logit becomes an order-preserving 32-bit key (NaN -> 0: never chosen).  The order is
// (logit descending, expert index ascending), so ties go to the lower index.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return __builtin_isnan(v) ? 0u : ord;
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// maximum over the wave (every lane gets it)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  m = max(m, dpp_u<kDppQuadXor1>(m));
  m = max(m, dpp_u<kDppQuadXor2>(m));
  m = max(m, dpp_u<kDppRowRor4>(m));
  m = max(m, dpp_u<kDppRowRor8>(m));
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)m, 0),
                         (uint32_t)__builtin_amdgcn_readlane((int)m, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)m, 32),
                         (uint32_t)__builtin_amdgcn_readlane((int)m, 48));
  return max(a, b);
}
// maximum / minimum over the first 16 lanes (returned to every lane)
__device__ __forceinline__ uint32_t row0_max_u32(uint32_t m) {
  m = max(m, dpp_u<kDppQuadXor1>(m));
  m = max(m, dpp_u<kDppQuadXor2>(m));
  m = max(m, dpp_u<kDppRowRor4>(m));
  m = max(m, dpp_u<kDppRowRor8>(m));
  return (uint32_t)__builtin_amdgcn_readlane((int)m, 0);
}
__device__ __forceinline__ int row0_min_i32(int m) {
  m = min(m, (int)dpp_u<kDppQuadXor1>((uint32_t)m));
  m = min(m, (int)dpp_u<kDppQuadXor2>((uint32_t)m));
  m = min(m, (int)dpp_u<kDppRowRor4>((uint32_t)m));
  m = min(m, (int)dpp_u<kDppRowRor8>((uint32_t)m));
  return __builtin_amdgcn_readlane(m, 0);
}

// Step 1: the k best of one wave's 128 logits (lane t holds expert indices base + 2t and
// base + 2t + 1).  Every lane returns the same keys (0 = none) and indices.
__device__ __forceinline__ void wave_candidates(float v0, float v1, int base, int lane,
                                                uint32_t (&ck)[kPK], int (&ci)[kPK]) {
  uint32_t k0 = order_key(v0), k1 = order_key(v1);
#pragma unroll
  for (int j = 0; j < kPK; ++j) {
    const uint32_t m = wave_max_u32(max(k0, k1));
    const uint64_t b0 = __ballot(m != 0u && k0 == m), b1 = __ballot(m != 0u && k1 == m);
    const int i0 = b0 ? 2 * __builtin_ctzll(b0) : 1 << 20;
    const int i1 = b1 ? 2 * __builtin_ctzll(b1) + 1 : 1 << 20;
    const int idx = i0 < i1 ? i0 : i1;
    ck[j] = m;
    ci[j] = m ? base + idx : -1;
    if (m && lane == (idx >> 1)) {
      if (idx & 1)
        k1 = 0u;
      else
        k0 = 0u;
    }
  }
}

// Step 2: the k best of the 16 candidates (4 waves x 4) held in lanes 0..15.  Every lane returns
// the same ids (-1 when fewer than j + 1 logits are selectable) and logit values.
__device__ __forceinline__ void merge_candidates(uint32_t key, int idx, int (&ids)[kPK],
                                                 float (&vals)[kPK]) {
#pragma unroll
  for (int j = 0; j < kPK; ++j) {
    const uint32_t m = row0_max_u32(key);
    const int pick = row0_min_i32((m != 0u && key == m) ? idx : (1 << 30));
    ids[j] = m ? pick : -1;
    vals[j] = m ? key_value(m) : 0.f;
    if (m && idx == pick) key = 0u;
  }
}

// ---- several row sums at once ----
// Sums each of v[0..7] over the 64 lanes.  Halving exchanges (lanes 32-63 against 0-31 with
// v_permlane32_swap, odd against even 16-lane rows with v_permlane16_swap, then 8-lane halves
// with a row rotation) leave lane l holding a partial of v[j(l)], j(l) = 4 bit3 + 2 bit4 + bit5
// of l; three adds within the 8-lane group finish it.  The lane with (l & 7) == 0 of each group
// returns its total for v[j(l)].
__device__ __forceinline__ int multi8_index(int lane) {
  return 4 * ((lane >> 3) & 1) + 2 * ((lane >> 4) & 1) + ((lane >> 5) & 1);
}
__device__ __forceinline__ float multi8_sum(const float (&v)[8], int lane) {
  float u[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2 * k]),
                                                    __float_as_uint(v[2 * k + 1]), false, false);
    u[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float w[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[2 * k]),
                                                    __float_as_uint(u[2 * k + 1]), false, false);
    w[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const bool hi8 = (lane & 8) != 0;
  const float keep = hi8 ? w[1] : w[0];
  const float give = hi8 ? w[0] : w[1];
  float z = keep + dpp_f<kDppRowRor8>(give);
  z += dpp_f<kDppRowHalfMirror>(z);
  z += dpp_f<kDppQuadXor1>(z);
  z += dpp_f<kDppQuadXor2>(z);
  return z;
}

// ---- weight rows ----
// Every weight load is a wave-uniform base (scalar registers) plus a 32-bit lane offset, so
// the per-lane part of each address costs one vector register.
template <typename T>
__device__ __forceinline__ T ld_nt_at(const uint8_t* base, uint32_t off) {
  typedef const __attribute__((address_space(1))) T* gp;
  return __builtin_nontemporal_load((gp)(base + off));
}
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Per-lane byte offsets, fixed for the whole launch.
struct LaneOff {
  uint32_t gu_sb;  // gate/up scale-or-bias: (lane & 1) * kGuMeta + (lane >> 1) * 2
  uint32_t dn_sb;  // down scale-or-bias: ((lane & 3) == 1) * kDnMeta + (lane >> 2) * 2
};

// Gate/up half row: 64 chunks of 16 bytes (32 codes, half a group).  Lane l of a wave that
// owns half hf reads chunk 64 hf + l; the even lane of each pair loads the group's scale,
// the odd lane its bias, and a lane swap gives each lane both.
struct HalfRow {
  v4u q;
  uint16_t sb;
};

__device__ __forceinline__ void load_half_row(HalfRow& r, const uint8_t* rec, int row, int hf,
                                              int lane, const LaneOff& o) {
  r.q = ld_nt_at<v4u>(rec + (size_t)row * (kPH / 2) + hf * 1024, (uint32_t)lane * 16u);
  r.sb = ld_nt_at<uint16_t>(rec + kGuCodes + (size_t)row * (kPH / kGroup * 2) + hf * 64, o.gu_sb);
}

__device__ __forceinline__ float half_row_partial(const HalfRow& r, const float* xc, float xsum,
                                                  int lane) {
  const float mine = bf16f(r.sb);
  const float other = dpp_f<kDppQuadXor1>(mine);
  const float s = (lane & 1) ? other : mine;
  const float bb = (lane & 1) ? mine : other;
  const uint4 q = make_uint4(r.q[0], r.q[1], r.q[2], r.q[3]);
  return (s * kCodeUnit) * dot_chunk_q4(q, xc) + bb * xsum;
}

// Down row: 1024 codes = 512 bytes; lane l reads codes 16 l .. 16 l + 15 (8 bytes).  Lane
// 4g loads group g's scale, lane 4g + 1 its bias; a quad broadcast gives both to all four.
struct DnRow {
  v2u q;
  uint16_t sb;
};

__device__ __forceinline__ void load_dn_row(DnRow& r, const uint8_t* slot, int row, int lane,
                                            const LaneOff& o) {
  const uint8_t* rec = slot + kDnOff;
  r.q = ld_nt_at<v2u>(rec + (size_t)row * (kPI / 2), (uint32_t)lane * 8u);
  r.sb = ld_nt_at<uint16_t>(rec + kDnCodes + (size_t)row * (kPI / kGroup * 2), o.dn_sb);
}

constexpr int kDppQuadBcast0 = 0x00;  // quad_perm [0,0,0,0]
constexpr int kDppQuadBcast1 = 0x55;  // quad_perm [1,1,1,1]

// sum(code_i * h_i) / 512 over 16 q4 codes in two words
__device__ __forceinline__ float dot8_q4(const v2u c, const float* __restrict__ h) {
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const uint32_t lo = c[d] & 0x0F0F0F0Fu;
    const uint32_t hi = (c[d] >> 4) & 0x0F0F0F0Fu;
    const float* hd = h + 8 * d;
    float q0, q2, q4, q6, q1, q3, q5, q7;
    codes2<false>(lo, q0, q2);
    codes2<true>(lo, q4, q6);
    codes2<false>(hi, q1, q3);
    codes2<true>(hi, q5, q7);
    acc0 = fmaf(q0, hd[0], acc0);
    acc1 = fmaf(q1, hd[1], acc1);
    acc0 = fmaf(q2, hd[2], acc0);
    acc1 = fmaf(q3, hd[3], acc1);
    acc0 = fmaf(q4, hd[4], acc0);
    acc1 = fmaf(q5, hd[5], acc1);
    acc0 = fmaf(q6, hd[6], acc0);
    acc1 = fmaf(q7, hd[7], acc1);
  }
  return acc0 + acc1;
}

__device__ __forceinline__ float dn_row_partial(const DnRow& r, const float* h, float hsum) {
  const float mine = bf16f(r.sb);
  const float s = dpp_f<kDppQuadBcast0>(mine);
  const float bb = dpp_f<kDppQuadBcast1>(mine);
  return (s * kCodeUnit) * dot8_q4(r.q, h) + bb * hsum;
}

// Loads of the next layer that do not depend on its routing: this wave's quarter of one of
// the workgroup's two router rows, and its gate and up half rows of the shared expert.
struct Prefetch {
  v4f rw[4];
  HalfRow sg, su;
};

__device__ __forceinline__ void issue_prefetch(Prefetch& p, const PLayer& L, int b, int wave,
                                               int lane, const LaneOff& o) {
  const uint8_t* wr = reinterpret_cast<const uint8_t*>(L.w_router) +
                      ((size_t)(2 * b + (wave >> 2)) * kPH + 1024 * (wave & 3)) * 4;
#pragma unroll
  for (int k = 0; k < 4; ++k) p.rw[k] = ld_nt_at<v4f>(wr + 1024 * k, (uint32_t)lane * 16u);
  const uint8_t* slot = L.base + (size_t)L.shared_slot * L.slot_bytes;
  const int row = 4 * b + (wave >> 1), hf = wave & 1;
  load_half_row(p.sg, slot, row, hf, lane, o);
  load_half_row(p.su, slot + kGuRec, row, hf, lane, o);
}

__global__ __launch_bounds__(kPT) void persist_kernel(PArgs a) {
  __shared__ __attribute__((aligned(16))) float xs[kPH];   // raw input of the current layer
  __shared__ __attribute__((aligned(16))) float hs[kNH];   // SwiGLU outputs of the 5 slots
  __shared__ float part_r[kCW];           // router partial per compute wave
  __shared__ float part_gu[kCW][10];      // gate/up partials: routed (2e, 2e+1), shared (8, 9)
  __shared__ float ydn[kPS][16];          // down outputs of this workgroup's 16 rows
  __shared__ float xsq[kXW], xsg[kXW];    // sum of squares / shared-gate dot partials
  __shared__ uint32_t cand_key[kXW * kPK];   // per exchange wave: its best logits' keys
  __shared__ int cand_idx[kXW * kPK];        // ... and expert indices
  __shared__ float s_w[kPK];
  __shared__ uint32_t s_epoch;
  __shared__ int s_abort;

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = a.n_layers;
  PersistWs xw = PersistWs::at(a.xw);

  if (tid == 0) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    s_abort = 0;
    const u32x4 e = xld<16>(rsrc(xw.ctl), 0);
    s_epoch = e.x;
    if ((int)(xcc & (kPX - 1)) != (b & (kPX - 1))) {
      s_abort = 1;
      atomicOr(xw.err, kPersistErrPlacement);
      if (a.dev_err) atomicOr(a.dev_err, kPersistErrPlacement);
    }
  }
  __syncthreads();
  const uint32_t epoch = s_epoch;

  if (wave < kCW) {
    // ================================ compute waves ================================
    LaneOff o;
    o.gu_sb = (uint32_t)(lane & 1) * (uint32_t)kGuMeta + (uint32_t)(lane >> 1) * 2u;
    o.dn_sb = ((lane & 3) == 1 ? (uint32_t)kDnMeta : 0u) + (uint32_t)(lane >> 2) * 2u;
    Prefetch pf;
    issue_prefetch(pf, a.layer[0], b, wave, lane, o);
    for (int L = 0; L < n; ++L) {
      const PLayer& Ly = a.layer[L];
      wg_barrier();  // A: xs holds the layer input
      {
        const int q = wave & 3;
        const float4* x4 = reinterpret_cast<const float4*>(xs) + 256 * q + lane;
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 xv = x4[64 * k];
          acc = fmaf(pf.rw[k][0], xv.x, acc);
          acc = fmaf(pf.rw[k][1], xv.y, acc);
          acc = fmaf(pf.rw[k][2], xv.z, acc);
          acc = fmaf(pf.rw[k][3], xv.w, acc);
        }
        acc = seg_sum<kWave>(acc);
        if (lane == 0) part_r[wave] = acc;
      }
      wg_barrier();  // B: router partials written
      // this wave's 32 inputs (raw; the RMS scale is applied to the finished dot products)
      const int hf = wave & 1;
      float xc[32];
      {
        const float4* x4 = reinterpret_cast<const float4*>(xs + 2048 * hf + 32 * lane);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float4 t = x4[v];
          xc[4 * v] = t.x;
          xc[4 * v + 1] = t.y;
          xc[4 * v + 2] = t.z;
          xc[4 * v + 3] = t.w;
        }
      }
      float xsum = 0.f;
#pragma unroll
      for (int c = 0; c < 32; ++c) xsum += xc[c];
      {
        const float g = seg_sum<kWave>(half_row_partial(pf.sg, xc, xsum, lane));
        const float u = seg_sum<kWave>(half_row_partial(pf.su, xc, xsum, lane));
        if (lane == 0) {
          part_gu[wave][8] = g;
          part_gu[wave][9] = u;
        }
      }
      wg_barrier();  // C: the routing candidates are in LDS
      int ids[kPK];
      {
        float vals[kPK];
        merge_candidates(lane < 16 ? cand_key[lane] : 0u, lane < 16 ? cand_idx[lane] : 0, ids,
                         vals);
      }
      // slot base of each routed expert (invalid ids read slot 0; their weight is 0)
      const uint8_t* slot[kPS];
#pragma unroll
      for (int e = 0; e < kPK; ++e) {
        const int id = __builtin_amdgcn_readfirstlane(ids[e]);
        slot[e] = Ly.base + (size_t)(id >= 0 && id < Ly.n_slots ? id : 0) * Ly.slot_bytes;
      }
      slot[kPK] = Ly.base + (size_t)Ly.shared_slot * Ly.slot_bytes;
      // routed gate/up half rows: this wave's row 4b + wave/2, half wave & 1
      const int gu_row = 4 * b + (wave >> 1);
      HalfRow gu[2 * kPK];
#pragma unroll
      for (int e = 0; e < kPK; ++e) {
        // (one row's codes and scale/bias stay together, so a row can be used as soon as
        // its own loads are back)
        load_half_row(gu[2 * e], slot[e], gu_row, hf, lane, o);
        issue_fence();
        load_half_row(gu[2 * e + 1], slot[e] + kGuRec, gu_row, hf, lane, o);
        issue_fence();
      }
      issue_fence();
      // Dot products as the rows arrive.  The down rows are issued only afterwards: loads of
      // one CU are served in issue order, so they would otherwise delay the gate/up rows.
      {
        float part[2 * kPK];
#pragma unroll
        for (int e = 0; e < 2 * kPK; ++e) part[e] = half_row_partial(gu[e], xc, xsum, lane);
        const float v = multi8_sum(part, lane);
        if ((lane & 7) == 0) part_gu[wave][multi8_index(lane)] = v;
      }
      issue_fence();
      // down rows: pairs p = 10 wave + i, expert p / 16, row 16 b + p % 16 (a wave spans at
      // most two experts)
      const int p0 = 10 * wave, e0 = p0 >> 4;
      const uint8_t* dslot0 = e0 == 0 ? slot[0] : e0 == 1 ? slot[1] : e0 == 2 ? slot[2]
                            : e0 == 3 ? slot[3] : slot[4];
      const uint8_t* dslot1 = e0 == 0 ? slot[1] : e0 == 1 ? slot[2] : e0 == 2 ? slot[3]
                            : slot[4];
      DnRow dn[10];
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int p = p0 + i;
        load_dn_row(dn[i], (p >> 4) == e0 ? dslot0 : dslot1, 16 * b + (p & 15), lane, o);
        issue_fence();
      }
      issue_fence();
      wg_barrier();  // D: gate/up partials written
      wg_barrier();  // E: hs holds h of all slots
      {
        const int p0 = 10 * wave;
        float h[16];
        float hsum = 0.f;
        float y[10];
#pragma unroll
        for (int i = 0; i < 10; ++i) {
          const int p = p0 + i, e = p >> 4;
          if (i == 0 || (p & 15) == 0) {
            const float4* h4 = reinterpret_cast<const float4*>(hs + e * kPI + 16 * lane);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float4 t = h4[v];
              h[4 * v] = t.x;
              h[4 * v + 1] = t.y;
              h[4 * v + 2] = t.z;
              h[4 * v + 3] = t.w;
            }
            hsum = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) hsum += h[c];
          }
          y[i] = dn_row_partial(dn[i], h, hsum);
        }
        float y8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y8[i] = y[i];
        const float s8 = multi8_sum(y8, lane);
        const float s9 = seg_sum<kWave>(y[8]);
        const float s10 = seg_sum<kWave>(y[9]);
        if ((lane & 7) == 0) {
          const int p = p0 + multi8_index(lane);
          ydn[p >> 4][p & 15] = s8;
        }
        if (lane == 0) {
          ydn[(p0 + 8) >> 4][(p0 + 8) & 15] = s9;
          ydn[(p0 + 9) >> 4][(p0 + 9) & 15] = s10;
        }
      }
      // The next layer's routing-independent rows (router quarter rows, shared gate/up half
      // rows) stream while this layer's output is exchanged, which the router waits for
      // anyway; issued earlier they would delay this CU's exchange loads queued behind them.
      // (The last layer re-reads its own rows: an unconditional issue keeps the compiler's
      // count of loads in flight exact.)
      issue_fence();
      issue_prefetch(pf, a.layer[L + 1 < n ? L + 1 : L], b, wave, lane, o);
      issue_fence();
      wg_barrier();  // F: down outputs written
    }
    wg_barrier();  // G: final gather done
  } else {
    // ================================ exchange waves ================================
    XCtx c;
    c.b = b;
    c.j = b / kPX;
    c.t = tid - kCW * kWave;
    {
      uint32_t xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      c.xcc = xcc;
    }
    c.abort = (lds_int*)&s_abort;
    c.err = xw.err;
    c.dev_err = a.dev_err;
    const int xwv = c.t >> 6;
    const auto r_out = rsrc(xw.g_out), r_lg = rsrc(xw.g_logit), r_h = rsrc(xw.g_h);
    float s = 0.f, sg = 0.f;
    // input of layer L (raw) into xs; partial sums of squares and of w_sg . x
    // w_sg: the layer's shared-gate vector, or the input vector itself (only the sum of
    // squares is then used)
    auto take_x = [&](const float (&v)[kNOut / kXT], const float* w_sg) {
      float2 w2[kNOut / kXT / 2];
#pragma unroll
      for (int i = 0; i < kNOut / kXT / 2; ++i)
        w2[i] = reinterpret_cast<const float2*>(w_sg)[c.t + kXT * i];
      float sq = 0.f, dg = 0.f;
#pragma unroll
      for (int i = 0; i < kNOut / kXT / 2; ++i) {
        const int p = c.t + kXT * i;
        xs[2 * p] = v[2 * i];
        xs[2 * p + 1] = v[2 * i + 1];
        sq = fmaf(v[2 * i], v[2 * i], sq);
        sq = fmaf(v[2 * i + 1], v[2 * i + 1], sq);
        dg = fmaf(w2[i].x, v[2 * i], dg);
        dg = fmaf(w2[i].y, v[2 * i + 1], dg);
      }
      sq = seg_sum<kWave>(sq);
      dg = seg_sum<kWave>(dg);
      if ((c.t & (kWave - 1)) == 0) {
        xsq[xwv] = sq;
        xsg[xwv] = dg;
      }
    };
    auto scale_of = [&](float eps) {
      const float ss = (xsq[0] + xsq[1]) + (xsq[2] + xsq[3]);
      return __builtin_amdgcn_rsqf(ss / (float)kPH + eps);
    };
    for (int L = 0; L < n; ++L) {
      const PLayer& Ly = a.layer[L];
      const uint32_t tag = epoch + (uint32_t)L + 1u;
      {
        float v[kNOut / kXT];
        if (L == 0) {
#pragma unroll
          for (int i = 0; i < kNOut / kXT / 2; ++i) {
            const float2 t = reinterpret_cast<const float2*>(a.x_in)[c.t + kXT * i];
            v[2 * i] = t.x;
            v[2 * i + 1] = t.y;
          }
        } else {
          gather<kNOut, kXT>(c, c.t, xw.g_out, xw.l_out, tag, v);
        }
        take_x(v, Ly.w_sg);
      }
      wg_barrier();  // A
      wg_barrier();  // B
      s = scale_of(a.eps);
      {
        const float d = (xsg[0] + xsg[1]) + (xsg[2] + xsg[3]);
        sg = sigmoidf_acc(s * d);
      }
      if (c.t < 2) {
        const float* pr = part_r + 4 * c.t;
        xst1(r_lg, 2 * b + c.t, s * ((pr[0] + pr[1]) + (pr[2] + pr[3])), tag);
      }
      // all 512 logits (thread t holds experts 2t, 2t+1); each exchange wave keeps the best
      // k of its 128 for the merge after the barrier
      {
        float v[2];
        gather<kNLogit, kXT>(c, c.t, xw.g_logit, xw.l_logit, tag, v);
        uint32_t ck[kPK];
        int ci[kPK];
        wave_candidates(v[0], v[1], 128 * xwv, c.t & (kWave - 1), ck, ci);
        if ((c.t & (kWave - 1)) < kPK) {
          const int j = c.t & (kWave - 1);
          uint32_t kk = ck[0];
          int ii = ci[0];
#pragma unroll
          for (int e = 1; e < kPK; ++e)
            if (j == e) {
              kk = ck[e];
              ii = ci[e];
            }
          cand_key[xwv * kPK + j] = kk;
          cand_idx[xwv * kPK + j] = ii;
        }
      }
      wg_barrier();  // C
      if (xwv == 0) {
        // routing weights (renormalised softmax over the selected) for the combine
        const int lane = c.t;
        int ids[kPK];
        float vals[kPK];
        merge_candidates(lane < 16 ? cand_key[lane] : 0u, lane < 16 ? cand_idx[lane] : 0, ids,
                         vals);
        float w[kPK], sum = 0.f;
#pragma unroll
        for (int e = 0; e < kPK; ++e) {
          w[e] = ids[e] >= 0 ? expf(vals[e] - vals[0]) : 0.f;
          sum += w[e];
        }
        const float inv = 1.f / sum;
        if (lane < kPK) {
          int id = ids[0];
          float we = w[0];
#pragma unroll
          for (int e = 1; e < kPK; ++e)
            if (lane == e) {
              id = ids[e];
              we = w[e];
            }
          s_w[lane] = (id >= 0 && id < Ly.n_slots) ? we * inv : 0.f;
          if (a.ids_trace && b == 0) a.ids_trace[L * kPK + lane] = id;
        }
      }
      wg_barrier();  // D
      if (c.t < 4 * kPS) {
        const int e = c.t >> 2, r = c.t & 3;
        const int gi = e < kPK ? 2 * e : 8;
        const float g = s * (part_gu[2 * r][gi] + part_gu[2 * r + 1][gi]);
        const float u = s * (part_gu[2 * r][gi + 1] + part_gu[2 * r + 1][gi + 1]);
        xst1(r_h, e * kPI + 4 * b + r, siluf_acc(g) * u, tag);
      }
      {
        float v[kNH / kXT];
        gather<kNH, kXT>(c, c.t, xw.g_h, xw.l_h, tag, v);
#pragma unroll
        for (int i = 0; i < kNH / kXT / 2; ++i) {
          const int p = c.t + kXT * i;
          hs[2 * p] = v[2 * i];
          hs[2 * p + 1] = v[2 * i + 1];
        }
      }
      wg_barrier();  // E
      wg_barrier();  // F
      if (c.t < 16) {
        const int row = 16 * b + c.t;
        float acc = xs[row];
#pragma unroll
        for (int e = 0; e < kPK; ++e) acc = fmaf(s_w[e], ydn[e][c.t], acc);
        acc = fmaf(sg, ydn[kPK][c.t], acc);
        xst1(r_out, row, acc, tag + 1u);
        if (L == n - 1) a.x_out[row] = acc;
      }
    }
    // RMSNorm of the stack output (every workgroup needs the full sum of squares)
    const uint32_t tag = epoch + (uint32_t)n + 1u;
    {
      float v[kNOut / kXT];
      gather<kNOut, kXT>(c, c.t, xw.g_out, xw.l_out, tag, v);
      take_x(v, a.layer[n - 1].w_sg);
    }
    wg_barrier();  // G
    if (a.xn_out && c.t < 16) {
      const float sn = scale_of(a.eps);
      const int row = 16 * b + c.t;
      a.xn_out[row] = xs[row] * sn;
    }
    if (b == 0 && c.t == 0) {
      u32x4 e;
      e.x = tag;
      e.y = e.z = e.w = 0;
      xst2<16>(rsrc(xw.ctl), 0, e);
    }
  }
}

}  // namespace

bool persist_shape_ok(const moe_layer* layers, int n_layers) {
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    if (L.experts.bits != 4 || L.experts.hidden != kPH || L.experts.inter != kPI ||
        L.experts.group != kGroup || L.n_experts != kPE || L.top_k != kPK ||
        L.shared_slot < 0 || !L.w_sg || L.experts.slot_bytes % 16 != 0)
      return false;
  }
  return n_layers >= 1;
}

bool persist_device_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  int cus = 0, coop = 0, xcc = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess ||
      hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess)
    return false;
  return cus == kPB && coop && xcc == kPX;
}

moe_status persist_launch(const moe_layer* layers, int n_layers, const float* x_in, float* x_out,
                          float* xn_out, float eps, int32_t* ids_trace, uint8_t* xw_base,
                          hipStream_t stream) {
  PArgs a{};
  a.n_layers = n_layers;
  a.eps = eps;
  a.x_in = x_in;
  a.x_out = x_out;
  a.xn_out = xn_out;
  a.ids_trace = ids_trace;
  a.xw = xw_base;
  a.dev_err = layers[0].experts.dev_err;
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    a.layer[l].base = reinterpret_cast<const uint8_t*>(L.experts.base);
    a.layer[l].w_router = L.w_router;
    a.layer[l].w_sg = L.w_sg;
    a.layer[l].slot_bytes = L.experts.slot_bytes;
    a.layer[l].n_slots = L.experts.n_slots;
    a.layer[l].shared_slot = L.shared_slot;
  }
  // A cooperative launch guarantees that all 256 workgroups are resident at once.  Tracing
  // tools that cannot follow cooperative launches get the same kernel through an ordinary
  // launch with MOE_PERSIST_PLAIN_LAUNCH=1: on an otherwise idle device the 256 workgroups
  // (one per CU) are still all resident; if they are not, the bounded waits report a timeout
  // through dev_err instead of hanging.
  static const bool plain = [] {
    const char* v = getenv("MOE_PERSIST_PLAIN_LAUNCH");
    return v && v[0] == '1';
  }();
  if (plain) {
    hipLaunchKernelGGL(persist_kernel, dim3(kPB), dim3(kPT), 0, stream, a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
  }
  void* args[] = {&a};
  const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(persist_kernel),
                                                  dim3(kPB), dim3(kPT), args, 0, stream);
  return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // namespace moe
