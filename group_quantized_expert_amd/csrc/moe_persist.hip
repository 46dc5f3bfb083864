// moe_persist.hip -- one launch per token: the whole q4 or q2 MoE layer stack decoded by a
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
// experts, top-4 plus one shared expert, q4 or q2 codes (the pages' 4-bit and 2-bit
// configurations, a2a-mcp.org, deep dive 3), group 64, bf16 scale and bias.  Other shapes use
// the kernel-per-step path in moe_decode.hip.  q2 runs the same schedule on half the bytes: a
// lane's 32 gate/up codes are 8 bytes instead of 16, spread into nibbles for the same integer
// products, and a down row is 256 bytes instead of 512.
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

#include <type_traits>

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

// record geometry (q4 or q2 codes, group 64)
template <int BITS>
struct PGeo {
  static constexpr size_t kGuCodes = (size_t)kPI * kPH * BITS / 8;    // 2 MiB (q4)
  static constexpr size_t kGuMeta = (size_t)kPI * (kPH / kGroup) * 2;  // 128 KiB (scale or bias)
  static constexpr size_t kGuRec = kGuCodes + 2 * kGuMeta;             // 2,359,296 (q4)
  static constexpr size_t kDnCodes = (size_t)kPH * kPI * BITS / 8;
  static constexpr size_t kDnMeta = (size_t)kPH * (kPI / kGroup) * 2;
  static constexpr size_t kDnOff = 2 * kGuRec;                         // down record in a slot
  static constexpr int kGuRow = kPH * BITS / 8;      // bytes of a gate/up row (2048 for q4)
  static constexpr int kGuLane = kGuRow / 2 / kWave;  // bytes per lane of a half row (16, 8)
  static constexpr int kDnRow = kPI * BITS / 8;      // bytes of a down row (512 for q4)
  static constexpr int kDnLane = kDnRow / kWave;     // bytes per lane of a down row (8, 4)
  static constexpr int kDnU4 = kDnRow / 16;          // 16-byte pieces of a down row
};

// exchange sizes (words)
constexpr int kNOut = kPH, kNLogit = kPE, kNH = kPS * kPI;
// copies of the SwiGLU words that the producers write, measured per width: q2 (ten packed
// words per workgroup, 20 KB per reader) gains from eight; q4 (five single-value words per
// row pair, 40 KB per reader) measured level or slower with four or eight, and keeps one
template <int BITS>
constexpr int kHCopies = BITS == 4 ? 1 : 8;
static_assert(kHCopies<4> <= (int)PersistWs::kGHCopies && kHCopies<2> <= (int)PersistWs::kGHCopies,
              "the exchange area holds at most kGHCopies copies");

struct PLayer {
  const uint8_t* base;
  const float* w_router;
  const float* w_router_cb;  // column-blocked copy [H/16][E][16], or null
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
#ifdef MOE_PHASE_STAMPS
  uint64_t* stamps;  // [layer][workgroup][kStampEvents] real-time counter values
#endif
};

// Phase time stamps, compiled in only by an instrumentation build (-DMOE_PHASE_STAMPS): lane 0
// of the wave that reaches event EV of layer L writes the GPU's 100 MHz real-time counter.
constexpr int kStampEvents = 32;
#ifdef MOE_PHASE_STAMPS
#define PHASE_STAMP(EV)                                                                       \
  do {                                                                                        \
    if (a.stamps && (threadIdx.x & (kWave - 1)) == 0)                                         \
      a.stamps[((size_t)L * kPB + blockIdx.x) * kStampEvents + (EV)] =                        \
          __builtin_amdgcn_s_memrealtime();                                                   \
  } while (0)
#else
#define PHASE_STAMP(EV) \
  do {                  \
  } while (0)
#endif

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
__device__ __forceinline__ void xst1(__amdgpu_buffer_rsrc_t r, int word, float v, uint32_t tag,
                                     int soff = 0) {
  u32x2 w;
  w.x = __float_as_uint(v);
  w.y = tag;
  __builtin_amdgcn_raw_buffer_store_b64(w, r, word * 8, soff, 16);
}

// q2 stacks: SwiGLU outputs travel two to a 64-bit word: each rounded to a 28-bit float (sign, exponent
// and 19 mantissa bits, to nearest even) in bits 0..27 and 28..55, and the low 8 bits of the
// layer tag in bits 56..63 (a word is at most one layer stale, so 8 bits tell fresh from old).
__device__ __forceinline__ uint64_t h28(float v) {
  const uint32_t u = __float_as_uint(v);
  return (uint64_t)((u + 7u + ((u >> 4) & 1u)) >> 4);
}
__device__ __forceinline__ void xst_h2(__amdgpu_buffer_rsrc_t r, int word, float v0, float v1,
                                       uint32_t tag, int soff) {
  const uint64_t w = h28(v0) | (h28(v1) << 28) | ((uint64_t)(tag & 0xFFu) << 56);
  u32x2 w2;
  w2.x = (uint32_t)w;
  w2.y = (uint32_t)(w >> 32);
  __builtin_amdgcn_raw_buffer_store_b64(w2, r, word * 8, soff, 16);
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

// Poll K 16-byte units p = t + kXT i of the SwiGLU buffer (two words, four values) until both
// words carry the layer's tag; returns the four values of each (zeros after an abort or a
// timeout).
template <int K>
__device__ __forceinline__ void poll_h(const XCtx& c, int t, __amdgpu_buffer_rsrc_t r,
                                       uint32_t tag, float4 (&v)[K]) {
  const uint32_t t8 = (tag & 0xFFu) << 24;
  const uint64_t t0 = now_ticks();
  while (true) {
    u32x4 w[K];
#pragma unroll
    for (int i = 0; i < K; ++i) w[i] = xld<16>(r, (t + kXT * i) * 16);
    bool ok = true;
#pragma unroll
    for (int i = 0; i < K; ++i)
      ok = ok && (w[i].y & 0xFF000000u) == t8 && (w[i].w & 0xFF000000u) == t8;
    if (ok) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        v[i].x = __uint_as_float(w[i].x << 4);
        v[i].y = __uint_as_float((w[i].x >> 28 | w[i].y << 4) << 4);
        v[i].z = __uint_as_float(w[i].z << 4);
        v[i].w = __uint_as_float((w[i].z >> 28 | w[i].w << 4) << 4);
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
  for (int i = 0; i < K; ++i) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
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

// Scale and bias rows.  A 2-byte gather per row costs the CU's memory queue nearly as much as a
// whole row of codes, so each wave fetches the scale/bias segments of all its rows of a phase
// with one 16-byte-per-lane gather, parks them in its own LDS area and reads its groups back.
// Gate/up half rows 0..7 (routed: expert e / 2, gate for even e, up for odd e) and 8, 9 (shared
// gate, up): chunks 0..3 hold the 32 scales of the half row, 4..7 its 32 biases.  Down rows
// (Down rows: chunks 0, 1 the 16 scales, 2, 3 the 16 biases, in the workgroup's down area.)
struct WaveMeta {
  uint4 gu[10][8];
};

__device__ __forceinline__ v4u ld_nt_ptr(const uint8_t* p) {
  typedef const __attribute__((address_space(1))) v4u* gp;
  return __builtin_nontemporal_load((gp)p);
}

// Gate/up half row: 64 chunks of 32 codes (16 bytes of q4, 8 of q2; half a group).  Lane l of
// a wave that owns half hf reads chunk 64 hf + l (inputs 2048 hf + 32 l .. + 31), which lies in
// group l / 2 of the half.
template <int BITS>
struct HalfRow {
  typename std::conditional<BITS == 4, v4u, v2u>::type q;
};

template <int BITS>
__device__ __forceinline__ void load_half_row(HalfRow<BITS>& r, const uint8_t* rec, int row,
                                              int hf, int lane) {
  using P = PGeo<BITS>;
  r.q = ld_nt_at<decltype(r.q)>(rec + (size_t)row * P::kGuRow + hf * (P::kGuRow / 2),
                                (uint32_t)lane * (uint32_t)P::kGuLane);
}

// address of 16-byte part `part` of the scale (seg 0) or bias (seg 1) segment of a gate/up
// half row
template <int BITS>
__device__ __forceinline__ const uint8_t* gu_meta_addr(const uint8_t* rec, int row, int hf,
                                                       int seg, int part) {
  using P = PGeo<BITS>;
  return rec + P::kGuCodes + (size_t)seg * P::kGuMeta + (size_t)row * (kPH / kGroup * 2) +
         hf * 64 + part * 16;
}

// ---- gate/up products as 4-bit integer dot products ----
// The layer input in fixed point: per group of 64 inputs an exponent E with 2^E above the group's
// largest magnitude, X = rint(x 2^(26 - E)), |X| <= 2^26 (a rounding step of at most 2^-27 of
// the group maximum, below fp32's own rounding of a typical element), split into seven signed hex
// digits (the hex digits of X + 0x8888888 are the digits plus 8).  Digit plane k of eight
// consecutive inputs packs their digit k, input j in bits 4j .. 4j + 3: the order in which
// v_dot8_i32_i4 pairs them with eight packed q4 codes (code j in bits 4j .. 4j + 3).  A code c
// enters as the signed nibble c ^ 8 = c - 8, so a chunk's sum of c x is
// unit * sum((c - 8) X) + 8 * sum(x),  unit = 2^(E - 26).
struct XDigits {
  uint4 plane[kXPlanes];  // the lane's 32 inputs (q4: dword d inputs 8d .. 8d + 7; q2: dwords
                          // 0, 1 the even, odd inputs of 0..15, dwords 2, 3 those of 16..31)
  float xsum;             // sum of the 32 inputs
  float unit;             // 2^(E - 26) of their group
};

template <int BITS>
__device__ __forceinline__ float half_row_partial(const HalfRow<BITS>& r, const uint4 (&meta)[8],
                                                  const XDigits& x, int lane) {
  const uint16_t* m = reinterpret_cast<const uint16_t*>(meta);
  const float s = bf16f(m[lane >> 1]);
  const float bb = bf16f(m[32 + (lane >> 1)]);
  v4u q;
  if constexpr (BITS == 4) {
    q = r.q;
  } else {
    // A word of 16 q2 codes (code j in bits 2j .. 2j + 1) masked with 0x33333333 leaves the even
    // codes as nibbles (code 2i in nibble i), shifted right by 2 first the odd ones: the q4
    // product then needs the digit planes of the inputs in the same order (q2 planes hold the
    // even inputs of each 16, then the odd ones).
    q[0] = r.q[0] & 0x33333333u;
    q[1] = (r.q[0] >> 2) & 0x33333333u;
    q[2] = r.q[1] & 0x33333333u;
    q[3] = (r.q[1] >> 2) & 0x33333333u;
  }
  return s * dot_chunk_q4_int(q, x.plane, x.xsum, x.unit) + bb * x.xsum;
}

// Down row: 1024 codes (512 bytes of q4, 256 of q2); lane l takes codes 16 l .. 16 l + 15
// (8 or 4 bytes), in group l / 4.
template <int BITS>
__device__ __forceinline__ const uint8_t* dn_meta_addr(const uint8_t* slot, int row, int seg,
                                                       int part) {
  using P = PGeo<BITS>;
  return slot + P::kDnOff + P::kDnCodes + (size_t)seg * P::kDnMeta +
         (size_t)row * (kPI / kGroup * 2) + part * 16;
}

constexpr int kDppQuadBcast0 = 0x00;  // quad_perm [0,0,0,0]
constexpr int kDppQuadBcast1 = 0x55;  // quad_perm [1,1,1,1]

// sum(code_i * h_i) / 512 over 16 q4 codes in two words
__device__ __forceinline__ float dot16_q4(const v2u c, const float* __restrict__ h) {
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

// sum(code_i * h_i) / 512 over 16 q2 codes in one word (code i at bits 2 i .. 2 i + 1)
__device__ __forceinline__ float dot16_q2(const uint32_t c, const float* __restrict__ h) {
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t f = (c >> (2 * m)) & 0x03030303u;  // byte j: code 4 j + m
    float q0, q1, q2, q3;
    codes2<false>(f, q0, q1);
    codes2<true>(f, q2, q3);
    acc0 = fmaf(q0, h[m], acc0);
    acc1 = fmaf(q1, h[4 + m], acc1);
    acc0 = fmaf(q2, h[8 + m], acc0);
    acc1 = fmaf(q3, h[12 + m], acc1);
  }
  return acc0 + acc1;
}

// The codes of a wave's first N0 down rows converted to floats ahead of barrier E (they do not
// depend on the SwiGLU outputs): qf[i][c] is code c of the lane's 16, times 2^-9, in the order
// the products below consume them; after E only the fused multiply-adds remain.
template <int BITS, int N0>
__device__ __forceinline__ void predecode_rows(const uint4 (*codes)[PGeo<BITS>::kDnU4], int p0,
                                               int lane, float (&qf)[N0][16]) {
#pragma unroll
  for (int i = 0; i < N0; ++i) {
    const uint8_t* cp = reinterpret_cast<const uint8_t*>(codes[p0 + i]) + PGeo<BITS>::kDnLane * lane;
    if constexpr (BITS == 4) {
      const uint2 q = *reinterpret_cast<const uint2*>(cp);
      const uint32_t w[2] = {q.x, q.y};
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t lo = w[d] & 0x0F0F0F0Fu, hi = (w[d] >> 4) & 0x0F0F0F0Fu;
        codes2<false>(lo, qf[i][8 * d + 0], qf[i][8 * d + 2]);
        codes2<true>(lo, qf[i][8 * d + 4], qf[i][8 * d + 6]);
        codes2<false>(hi, qf[i][8 * d + 1], qf[i][8 * d + 3]);
        codes2<true>(hi, qf[i][8 * d + 5], qf[i][8 * d + 7]);
      }
    } else {
      const uint32_t c = *reinterpret_cast<const uint32_t*>(cp);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t f = (c >> (2 * m)) & 0x03030303u;
        codes2<false>(f, qf[i][m], qf[i][4 + m]);
        codes2<true>(f, qf[i][8 + m], qf[i][12 + m]);
      }
    }
  }
}
// the products of dot16_q4 / dot16_q2 on pre-converted codes, in the same order
template <int BITS>
__device__ __forceinline__ float dot16_pre(const float (&q)[16], const float* __restrict__ h) {
  float acc0 = 0.f, acc1 = 0.f;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        acc0 = fmaf(q[8 * d + k], h[8 * d + k], acc0);
        acc1 = fmaf(q[8 * d + k + 1], h[8 * d + k + 1], acc1);
      }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc0 = fmaf(q[m], h[m], acc0);
      acc1 = fmaf(q[4 + m], h[4 + m], acc1);
      acc0 = fmaf(q[8 + m], h[8 + m], acc0);
      acc1 = fmaf(q[12 + m], h[12 + m], acc1);
    }
  }
  return acc0 + acc1;
}

// Lane partials of N consecutive down rows p0 .. p0 + N - 1 (row p: slot p / 16, row 16 g + p % 16)
// from the rows parked in LDS and the SwiGLU outputs hs
template <int BITS, int N, int N0 = 0>
__device__ __forceinline__ void down_partials(const float* hs,
                                              const uint4 (*codes)[PGeo<BITS>::kDnU4],
                                              const uint4 (*meta)[4], int p0, int lane,
                                              float (&y)[N], const float (&qf)[N0 > 0 ? N0 : 1][16] = {}) {
  float h[16];
  float hsum = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
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
    // (meta: the row's 16 scales then 16 biases)
    const uint16_t* m = reinterpret_cast<const uint16_t*>(meta[p]);
    const float s = bf16f(m[lane >> 2]);
    const float bb = bf16f(m[16 + (lane >> 2)]);
    const uint8_t* cp = reinterpret_cast<const uint8_t*>(codes[p]) + PGeo<BITS>::kDnLane * lane;
    float d;
    if (i < N0) {
      d = dot16_pre<BITS>(qf[i < N0 ? i : 0], h);
    } else if constexpr (BITS == 4) {
      const uint2 q = *reinterpret_cast<const uint2*>(cp);
      v2u c;
      c[0] = q.x;
      c[1] = q.y;
      d = dot16_q4(c, h);
    } else {
      d = dot16_q2(*reinterpret_cast<const uint32_t*>(cp), h);
    }
    y[i] = (s * kCodeUnit) * d + bb * hsum;
  }
}

// ---- the K-split router ----
// Workgroup b owns the 16 output rows of row group g(b) = 32 (b mod 8) + b / 8 (adjacent groups,
// and so the two halves of each 128-byte router line, stay on one XCD).  At the end of a layer it
// multiplies its 16 finished output values by the matching 16 router columns of the next layer,
// giving a partial sum for every expert; the all-reduce of these partials over the 256
// workgroups is the next layer's router GEMV, with the RMS scale applied afterwards:
// logits = s * W_r x = W_r (s x).
__device__ __forceinline__ int row_group(int b) { return 32 * (b & (kPX - 1)) + (b >> 3); }

// A partial vector: the 512 logit partials, then the sum of squares of the workgroup's rows and
// their dot with the shared-expert gate, as 257 tagged pairs.  Slice j (pairs 9 j .. 9 j + 8,
// the last slice short) is reduced by the workgroups with b / 8 == j.
constexpr int kNPart = 514;
constexpr int kPartSq = 512, kPartSg = 513;
constexpr int kPartPairs = kNPart / 2;  // 257
constexpr int kSliceP = 9;
static_assert(kPJ * kSliceP >= kPartPairs && kPJ * (kSliceP - 1) < kPartPairs, "");

// pair index of the level-1 area: XCD x, slice j, pair i of the slice, producer q of the XCD
__device__ __forceinline__ int p1_pair(int x, int j, int i, int q) {
  return ((x * kPJ + j) * kSliceP + i) * kPJ + q;
}
// pair index of the level-2 area: slice j, pair i of the slice, XCD x
__device__ __forceinline__ int g2_pair(int j, int i, int x) { return (j * kSliceP + i) * kPX + x; }

// Loads of the next layer that do not depend on its routing, issued by each compute wave
// during the down products: its gate and up half rows of the shared expert.
template <int BITS>
struct Prefetch {
  v4u meta;  // lanes 0..15: half row l / 8 (gate, up), segment (l / 4) & 1, part l & 3
  HalfRow<BITS> sg, su;
};

template <int BITS>
__device__ __forceinline__ void issue_prefetch(Prefetch<BITS>& p, const PLayer& L, int b,
                                               int wave, int lane) {
  using P = PGeo<BITS>;
  const uint8_t* slot = L.base + (size_t)L.shared_slot * L.slot_bytes;
  const int row = 4 * b + (wave >> 1), hf = wave & 1;
  const int ml = lane & 15;
  p.meta = ld_nt_ptr(
      gu_meta_addr<BITS>(slot + (ml >> 3) * P::kGuRec, row, hf, (ml >> 2) & 1, ml & 3));
  load_half_row<BITS>(p.sg, slot, row, hf, lane);
  load_half_row<BITS>(p.su, slot + P::kGuRec, row, hf, lane);
}

// The next layer's router columns of this workgroup's 16 rows, read by the exchange waves one
// 64-byte segment per 4 lanes: exchange wave v, lane l, step k holds columns 16 g + 4 (l & 3)
// .. + 3 of expert 128 v + 16 k + l / 4.  Lanes 0..15 of the last exchange wave also hold the
// shared-gate weights of the 16 rows.
struct RouterCols {
  v4f w[8];
  float sg;
};

__device__ __forceinline__ void issue_router_cols(RouterCols& rc, const PLayer& L, int g, int xwv,
                                                  int xl) {
  // block g of the column-blocked copy: experts 128 xwv + 16 k + l / 4 are 1 KB contiguous per
  // step; in the plain layout the same registers come from 16 rows of 64 bytes per step
  const bool cb = L.w_router_cb != nullptr;
  const uint32_t gu = __builtin_amdgcn_readfirstlane(g), wu = __builtin_amdgcn_readfirstlane(xwv);
  const uint8_t* wr =
      cb ? reinterpret_cast<const uint8_t*>(L.w_router_cb) + (gu * kPE + 128u * wu) * 64u
         : reinterpret_cast<const uint8_t*>(L.w_router) + (128u * wu * kPH + 16u * gu) * 4u;
  const size_t step = cb ? 1024 : (size_t)16 * kPH * 4;
  const uint32_t off = cb ? (uint32_t)xl * 16u
                          : (uint32_t)(xl >> 2) * (uint32_t)(kPH * 4) + (uint32_t)(xl & 3) * 16u;
#pragma unroll
  for (int k = 0; k < 8; ++k) rc.w[k] = ld_nt_at<v4f>(wr + step * k, off);
  rc.sg = xwv == kXW - 1 ? ld_nt_at<float>(reinterpret_cast<const uint8_t*>(L.w_sg) + (size_t)16 * g * 4,
                                     (uint32_t)(xl & 15) * 4u)
                   : 0.f;
}

constexpr int kDppRowShl4 = 0x104;  // row_shl:4: lane i of each row <- lane i + 4

typedef __attribute__((address_space(3))) uint32_t lds_u32;

// Exchange-wave barrier (the four exchange waves only): an LDS counter, bounded wait.
__device__ __forceinline__ void x_barrier(const XCtx& c, lds_u32* ctr, uint32_t& gen) {
  gen += kXW;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if ((c.t & (kWave - 1)) == 0)
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const uint64_t t0 = now_ticks();
  while (*(volatile lds_u32*)ctr < gen) {
    if (now_ticks() - t0 > kSpinTicks) {
      fail(c, kPersistErrTimeout);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}

// Compute waves wait for LDS words that exchange waves set after writing the data they guard:
// a flag equal to the layer's tag, or a counter reaching a target.  Bounded (the exchange waves
// always set them, also after a failed exchange, so the bound is only a safety net).
__device__ __forceinline__ void wait_flag(lds_u32* f, uint32_t tag) {
  const uint64_t t0 = now_ticks();
  while (*(volatile lds_u32*)f != tag) {
    if (now_ticks() - t0 > kSpinTicks) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_count(lds_u32* f, uint32_t target) {
  const uint64_t t0 = now_ticks();
  while (*(volatile lds_u32*)f < target) {
    if (now_ticks() - t0 > kSpinTicks) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void set_flag(lds_u32* f, uint32_t tag) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  *(volatile lds_u32*)f = tag;
}
// one increment per calling wave, after the wave's LDS writes have landed
__device__ __forceinline__ void add_count(lds_u32* f, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) __hip_atomic_fetch_add(f, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Poll K tagged pairs per lane until both tags of every active pair equal tag (inactive pairs
// are not read and return zeros).  Bounded: a timeout raises the abort flag.
// SLEEP: s_sleep argument between rounds (0: poll back to back)
template <int K, int AUX, int SLEEP = 0>
__device__ __forceinline__ void poll_set(const XCtx& c, __amdgpu_buffer_rsrc_t r,
                                         const int (&pair)[K], const bool (&act)[K],
                                         uint32_t tag, float (&v)[2 * K]) {
#pragma unroll
  for (int i = 0; i < 2 * K; ++i) v[i] = 0.f;
  if (*(volatile lds_int*)c.abort) return;
  const uint64_t t0 = now_ticks();
  while (true) {
    u32x4 w[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (act[i]) {
        w[i] = xld<AUX>(r, pair[i] * 16);
      } else {
        w[i].x = w[i].z = 0u;
        w[i].y = w[i].w = tag;
      }
    }
    bool ok = true;
#pragma unroll
    for (int i = 0; i < K; ++i) ok = ok && w[i].y == tag && w[i].w == tag;
    if (ok) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        v[2 * i] = __uint_as_float(w[i].x);
        v[2 * i + 1] = __uint_as_float(w[i].z);
      }
      return;
    }
    if (*(volatile lds_int*)c.abort) return;
    if (now_ticks() - t0 > kSpinTicks) {
      fail(c, kPersistErrTimeout);
      return;
    }
    if (SLEEP) __builtin_amdgcn_s_sleep(SLEEP);
  }
}

__device__ __forceinline__ int wave_min_i32(int m) {
  m = min(m, (int)dpp_u<kDppQuadXor1>((uint32_t)m));
  m = min(m, (int)dpp_u<kDppQuadXor2>((uint32_t)m));
  m = min(m, (int)dpp_u<kDppRowRor4>((uint32_t)m));
  m = min(m, (int)dpp_u<kDppRowRor8>((uint32_t)m));
  const int a = min(__builtin_amdgcn_readlane(m, 0), __builtin_amdgcn_readlane(m, 16));
  const int b = min(__builtin_amdgcn_readlane(m, 32), __builtin_amdgcn_readlane(m, 48));
  return min(a, b);
}

// maximum over the wave, in every lane, without scalar round trips: two quad steps and a
// half-row mirror give the 8-lane maximum, a row rotation the 16-lane one, then 16- and
// 32-lane swaps combine the four rows.
__device__ __forceinline__ uint32_t wave_max_all(uint32_t m) {
  m = max(m, dpp_u<kDppQuadXor1>(m));
  m = max(m, dpp_u<kDppQuadXor2>(m));
  m = max(m, dpp_u<kDppRowHalfMirror>(m));
  m = max(m, dpp_u<kDppRowRor8>(m));
  const auto r16 = __builtin_amdgcn_permlane16_swap(m, m, false, false);
  m = max(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  return max(r32[0], r32[1]);
}

// Top-4 of the 512 logits on one wave (lane l holds expert 128 (m >> 1) + 2 l + (m & 1) in
// v[m]); order: logit descending, expert index ascending (ties go to the lower index), NaN never
// chosen.  Every lane returns the same ids (-1 when fewer than j + 1 logits are selectable) and
// logit values; a tie across lanes falls back to the smallest expert index over the tied lanes.
// Each lane first sorts its eight candidates once (a 19-comparator network on 64-bit keys: the
// order-preserving logit key, then 7 - m, so equal logits in a lane order by index); each of the
// four rounds then takes the wave maximum of the lanes' heads and the lane that owns the winner
// drops its head, instead of rescanning its eight candidates in a dependent chain.
__device__ __forceinline__ void wave_topk512(const float (&v)[8], int lane, int (&ids)[kPK],
                                             float (&vals)[kPK]) {
  uint64_t k[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) k[m] = ((uint64_t)order_key(v[m]) << 3) | (uint64_t)(7 - m);
  auto ce = [&](int i, int j) {  // k[i] >= k[j] afterwards
    const bool sw = k[j] > k[i];
    const uint64_t hi = sw ? k[j] : k[i], lo = sw ? k[i] : k[j];
    k[i] = hi;
    k[j] = lo;
  };
  // Batcher's odd-even merge sort of 8
  ce(0, 1); ce(2, 3); ce(4, 5); ce(6, 7);
  ce(0, 2); ce(1, 3); ce(4, 6); ce(5, 7);
  ce(1, 2); ce(5, 6);
  ce(0, 4); ce(1, 5); ce(2, 6); ce(3, 7);
  ce(2, 4); ce(3, 5);
  ce(1, 2); ce(3, 4); ce(5, 6);
  uint64_t h0 = k[0], h1 = k[1], h2 = k[2], h3 = k[3];
#pragma unroll
  for (int j = 0; j < kPK; ++j) {
    const uint32_t bk = (uint32_t)(h0 >> 3);  // 0 once the lane has nothing left (NaN keys are 0)
    const int bm = 7 - (int)(h0 & 7);
    const uint32_t top = wave_max_all(bk);
    const int my_idx = 128 * (bm >> 1) + 2 * lane + (bm & 1);
    const uint64_t hold = __ballot(top != 0u && bk == top);
    int pick = -1;
    if (hold) {
      if ((hold & (hold - 1)) == 0) {
        pick = __builtin_amdgcn_readlane(my_idx, __builtin_ctzll(hold));
      } else {
        pick = wave_min_i32(bk == top ? my_idx : (1 << 30));
      }
    }
    ids[j] = pick;
    vals[j] = hold ? key_value(top) : 0.f;
    const bool won = hold && my_idx == pick;
    h0 = won ? h1 : h0;
    h1 = won ? h2 : h1;
    h2 = won ? h3 : h2;
    h3 = won ? 0ull : h3;
  }
}

template <int BITS>
__global__ __launch_bounds__(kPT) void persist_kernel(PArgs a) {
  using P = PGeo<BITS>;
  __shared__ __attribute__((aligned(16))) float xs[kPH];   // raw input of the current layer
  __shared__ __attribute__((aligned(16))) float hs[kNH];   // SwiGLU outputs of the 5 slots
  __shared__ float part_gu[kCW][10];      // gate/up partials: routed (2e, 2e+1), shared (8, 9)
  __shared__ float ydn[kPS][16];          // down outputs of this workgroup's 16 rows
  __shared__ WaveMeta wmeta[kCW];         // per compute wave: scale/bias of its gate/up rows
  // the layer input as digit planes: chunk 64 hf + l = inputs 2048 hf + 32 l .. + 31
  __shared__ uint4 xdig[2 * kWave][kXPlanes];
  __shared__ float2 xaux[2 * kWave];       // per chunk: sum of its inputs, digit unit
  // the workgroup's 80 down rows (pair p: slot p / 16, row 16 g + p % 16): codes and
  // scale/bias, loaded by the exchange waves
  __shared__ __attribute__((aligned(16))) uint4 dn_codes[kPS * 16][P::kDnU4];
  __shared__ uint4 dn_meta[kPS * 16][4];
  __shared__ float xsq[kXW];
  __shared__ int s_ids[kPK];
  __shared__ float s_w[kPK];
  __shared__ float s_scale, s_sg;
  __shared__ uint32_t flag_ids, flag_w, flag_x, flag_xd, xbar, xread, gu_issued, dn_parked;
  __shared__ uint32_t h_pair[kCW / 2];     // gate/up halves finished per row, 2 per layer
  __shared__ uint32_t h_rows;              // q2: rows of h finished, 4 per layer
  __shared__ float h_stage[kCW / 2][kPS];  // q2: this workgroup's h, row 4b + r, slot e
  __shared__ uint32_t s_epoch;
  __shared__ int s_abort;

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = a.n_layers;
  const int g = row_group(b);
  PersistWs xw = PersistWs::at(a.xw);

  if (tid == 0) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    s_abort = 0;
    flag_ids = 0;
    flag_w = 0;
    flag_x = 0;
    flag_xd = 0;
    xbar = 0;
    xread = 0;
    gu_issued = 0;
    dn_parked = 0;
    for (int r = 0; r < kCW / 2; ++r) h_pair[r] = 0;
    h_rows = 0;
    const u32x4 e = xld<16>(rsrc(xw.ctl), 0);
    s_epoch = e.x;
    if ((int)(xcc & (kPX - 1)) != (b & (kPX - 1))) {
      s_abort = 1;
      atomicOr(xw.err, kPersistErrPlacement);
      if (a.dev_err) atomicOr(a.dev_err, kPersistErrPlacement);
    }
  }
  __syncthreads();
  const uint32_t epoch = __builtin_amdgcn_readfirstlane(s_epoch);

  // one output row of this workgroup: residual + routed experts + gated shared expert
  auto out_row = [&](int r) {
    float acc = xs[16 * g + r];
#pragma unroll
    for (int e = 0; e < kPK; ++e) acc = fmaf(s_w[e], ydn[e][r], acc);
    return fmaf(s_sg, ydn[kPK][r], acc);
  };

  if (wave < kCW) {
    // ================================ compute waves ================================
    const int hf = wave & 1;
    WaveMeta& wm = wmeta[wave];
    Prefetch<BITS> pf;
    issue_prefetch<BITS>(pf, a.layer[0], b, wave, lane);
    for (int L = 0; L < n; ++L) {
      // per-lane values are rebuilt every layer from an opaque copy of the lane index, so
      // that the compiler does not hold loop-invariant lane addresses across the layer loop
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const PLayer& Ly = a.layer[L];
      const uint32_t tag = epoch + (uint32_t)L + 1u;
      wait_flag((lds_u32*)&flag_ids, tag);
      // slot base of each routed expert (invalid ids read slot 0; their weight is 0)
      const uint8_t* slot[kPS];
#pragma unroll
      for (int e = 0; e < kPK; ++e) {
        const int id = __builtin_amdgcn_readfirstlane(s_ids[e]);
        slot[e] = Ly.base + (size_t)(id >= 0 && id < Ly.n_slots ? id : 0) * Ly.slot_bytes;
      }
      slot[kPK] = Ly.base + (size_t)Ly.shared_slot * Ly.slot_bytes;
      // routed gate/up half rows: this wave's row 4b + wave/2, half wave & 1; first the
      // scale/bias of all eight (lane l: half row l / 8, segment (l / 4) & 1, part l & 3)
      const int gu_row = 4 * b + (wave >> 1);
      v4u gmeta;
      {
        const int me = ln >> 3, ms = me >> 1;
        const uint8_t* mrec = (ms == 0 ? slot[0] : ms == 1 ? slot[1] : ms == 2 ? slot[2] : slot[3]) +
                              (size_t)(me & 1) * P::kGuRec;
        gmeta = ld_nt_ptr(gu_meta_addr<BITS>(mrec, gu_row, hf, (ln >> 2) & 1, ln & 3));
      }
      issue_fence();
      HalfRow<BITS> gu[2 * kPK];
#pragma unroll
      for (int e = 0; e < kPK; ++e) {
        load_half_row<BITS>(gu[2 * e], slot[e], gu_row, hf, ln);
        issue_fence();
        load_half_row<BITS>(gu[2 * e + 1], slot[e] + P::kGuRec, gu_row, hf, ln);
        issue_fence();
      }
      add_count((lds_u32*)&gu_issued, ln);
      // The second compute wave on each SIMD (waves 4..7) issued its rows after the first, so its
      // rows arrive last; with the default arbitration by age it would also get the VALU last and
      // its row pairs would publish their SwiGLU outputs ~1.5 us after the others.  A raised issue
      // priority until its products are done lets it work on its rows as they come in.
      if (wave >= kCW / 2) __builtin_amdgcn_s_setprio(1);
      if (wave == 0) PHASE_STAMP(5);
      // down rows of this wave (in LDS after barrier E): pairs p = 8 wave + i
      const int p0 = 8 * wave;
      wait_count((lds_u32*)&flag_xd, (uint32_t)(kXW - 1) * (uint32_t)(L + 1));
      if (wave == 0) PHASE_STAMP(6);
      // this lane's 32 inputs (raw; the RMS scale is applied to the finished dot products)
      XDigits xc;
      {
        const int ch = kWave * hf + ln;
#pragma unroll
        for (int k = 0; k < kXPlanes; ++k) xc.plane[k] = xdig[ch][k];
        const float2 au = xaux[ch];
        xc.xsum = au.x;
        xc.unit = au.y;
      }
      // park the scale/bias segments in this wave's LDS area (same-wave reads below see them)
      if (ln < 16) wm.gu[8 + (ln >> 3)][((ln >> 2) & 1) * 4 + (ln & 3)] =
          make_uint4(pf.meta[0], pf.meta[1], pf.meta[2], pf.meta[3]);
      wm.gu[ln >> 3][((ln >> 2) & 1) * 4 + (ln & 3)] = make_uint4(gmeta[0], gmeta[1], gmeta[2], gmeta[3]);
      {
        const float gs = seg_sum<kWave>(half_row_partial(pf.sg, wm.gu[8], xc, ln));
        const float us = seg_sum<kWave>(half_row_partial(pf.su, wm.gu[9], xc, ln));
        if (ln == 0) {
          part_gu[wave][8] = gs;
          part_gu[wave][9] = us;
        }
      }
      {
        float part[2 * kPK];
#pragma unroll
        for (int e = 0; e < 2; ++e) part[e] = half_row_partial(gu[e], wm.gu[e], xc, ln);
#pragma unroll
        for (int e = 2; e < 4; ++e) part[e] = half_row_partial(gu[e], wm.gu[e], xc, ln);
#pragma unroll
        for (int e = 4; e < 6; ++e) part[e] = half_row_partial(gu[e], wm.gu[e], xc, ln);
#pragma unroll
        for (int e = 6; e < 8; ++e) part[e] = half_row_partial(gu[e], wm.gu[e], xc, ln);
        const float v = multi8_sum(part, ln);
        if ((ln & 7) == 0) part_gu[wave][multi8_index(ln)] = v;
      }
      if (wave == 0) PHASE_STAMP(7);
      {
        // row 4b + wave/2 is split over this wave and its pair: whichever finishes second
        // (its count is odd) combines the halves and publishes h of the row for the 5 slots
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        uint32_t old = 0;
        if (ln == 0)
          old = __hip_atomic_fetch_add(&h_pair[wave >> 1], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
        old = __builtin_amdgcn_readfirstlane(old);
        if constexpr (BITS == 4) {
          if (old == 2u * (uint32_t)L + 1u && ln < kPS) {
            const int r = wave >> 1, gi = ln < kPK ? 2 * ln : 8;
            wait_flag((lds_u32*)&flag_w, tag);  // the RMS scale (set right after the ids)
            const float s = s_scale;
            const float gg = s * (part_gu[2 * r][gi] + part_gu[2 * r + 1][gi]);
            const float u = s * (part_gu[2 * r][gi + 1] + part_gu[2 * r + 1][gi + 1]);
            const auto rh = rsrc(xw.g_h);
            const float hv = siluf_acc(gg) * u;
#pragma unroll
            for (int cp = 0; cp < kHCopies<BITS>; ++cp)
              xst1(rh, ln * kPI + 4 * b + r, hv, tag, cp * (int)PersistWs::kGHCopy);
          }
        } else if (old == 2u * (uint32_t)L + 1u) {
          // q2: the row's values go to LDS; the wave that finishes the workgroup's fourth row
          // publishes all 20, two per 64-bit word
          const int r = wave >> 1;
          if (ln < kPS) {
            const int gi = ln < kPK ? 2 * ln : 8;
            wait_flag((lds_u32*)&flag_w, tag);
            const float s = s_scale;
            const float gg = s * (part_gu[2 * r][gi] + part_gu[2 * r + 1][gi]);
            const float u = s * (part_gu[2 * r][gi + 1] + part_gu[2 * r + 1][gi + 1]);
            h_stage[r][ln] = siluf_acc(gg) * u;
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          uint32_t done = 0;
          if (ln == 0)
            done = __hip_atomic_fetch_add(&h_rows, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_WORKGROUP);
          done = __builtin_amdgcn_readfirstlane(done);
          if (done == 4u * (uint32_t)L + 3u && ln < 2 * kPS) {
            const int e = ln >> 1, r0 = 2 * (ln & 1);
            const auto rh = rsrc(xw.g_h);
            const float h0 = h_stage[r0][e], h1 = h_stage[r0 + 1][e];
#pragma unroll
            for (int cp = 0; cp < kHCopies<BITS>; ++cp)
              xst_h2(rh, e * (kPI / 2) + 2 * b + (ln & 1), h0, h1, tag, cp * (int)PersistWs::kGHCopy);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // While the exchange waves gather the SwiGLU outputs, convert the codes of this wave's
      // first kPreRows down rows (parked in LDS by then) to floats (measured per 60-layer token:
      // four rows 821.4 us, all eight 824.0, none 826.8).
      wait_count((lds_u32*)&dn_parked, (uint32_t)kXW * (uint32_t)(L + 1));
      constexpr int kPreRows = 4;
      float qf[kPreRows][16];
      predecode_rows<BITS, kPreRows>(dn_codes, p0, ln, qf);
      // keep the conversions ahead of the barrier (the scheduler would sink them to their use)
#pragma unroll
      for (int i = 0; i < kPreRows; ++i)
#pragma unroll
        for (int c = 0; c < 16; ++c) asm volatile("" : "+v"(qf[i][c]));
      if (wave == 0) PHASE_STAMP(8);
      wg_barrier();  // E: hs holds h of all slots
      {
        // the routed slots' 64 rows, 8 per compute wave (the shared slot's 16 rows go to the
        // exchange waves, a third wave per SIMD during the down products)
        float y[8];
        down_partials<BITS, 8, kPreRows>(hs, dn_codes, dn_meta, p0, ln, y, qf);
        const float s8 = multi8_sum(y, ln);
        if ((ln & 7) == 0) {
          const int p = p0 + multi8_index(ln);
          ydn[p >> 4][p & 15] = s8;
        }
      }
      // The next layer's routing-independent rows, issued after this wave's products (an issue
      // into the CU's full memory queue would stall the wave) and behind the next layer's router
      // columns, which the exchange waves issue at barrier E: those are needed first, by this
      // layer's publish.  (The last layer re-reads its own rows: an unconditional issue keeps the
      // compiler's count of loads in flight exact.)
      issue_fence();
      issue_prefetch<BITS>(pf, a.layer[L + 1 < n ? L + 1 : L], b, wave, ln);
      issue_fence();
      if (wave == 0) PHASE_STAMP(12);
      wg_barrier();  // F: down outputs written
    }
  } else {
    // ================================ exchange waves ================================
    // Wave 0 carries the routing (all-reduce hops 2 and 3, top-k); waves 1..3 fill xs (wave 2
    // also fetches this workgroup's slice of the layer input); all four take part in hop 1 and
    // in the SwiGLU all-gather.
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
    const int xwv = wave - kCW, xl = c.t & (kWave - 1);
    const int x = (int)(c.xcc & (kPX - 1));
    uint32_t xgen = 0;
    lds_u32* bar = (lds_u32*)&xbar;
    const auto r_out = rsrc(xw.g_out), r_p1 = rsrc(xw.p1), r_g2 = rsrc(xw.g2);
    const auto r_lout = rsrc(xw.l_out + (size_t)x * kNOut);
    const auto r_lpart = rsrc(reinterpret_cast<uint8_t*>(xw.l_part) +
                              (size_t)x * PersistWs::kLPart);
    // The partial vector of the next layer from this workgroup's 16 rows (value of row r in
    // lane r of each 16-lane row), published into this XCD's level-1 area (plain stores: only
    // this XCD reads it).  Thread t: experts 2t, 2t + 1; lane 0 of the last exchange wave also
    // the sum of squares and the shared-gate dot.
    RouterCols rc;
    // ow: rows 4 (l & 3) .. 4 (l & 3) + 3 of the 16 (the lane's router columns); ov: row l & 15
    auto publish_part = [&](const float4 ow, float ov, uint32_t tag, int xl) {
      // expert 128 xwv + 16 k + l / 4: a 4-lane sum; lanes 8u then pair experts 2u, 2u + 1.
      // The eight sums are independent: built side by side, then stored together.
      float p[8], odd[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        p[k] = rc.w[k][0] * ow.x;
        p[k] = fmaf(rc.w[k][1], ow.y, p[k]);
        p[k] = fmaf(rc.w[k][2], ow.z, p[k]);
        p[k] = fmaf(rc.w[k][3], ow.w, p[k]);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) p[k] += dpp_f<kDppQuadXor1>(p[k]);
#pragma unroll
      for (int k = 0; k < 8; ++k) p[k] += dpp_f<kDppQuadXor2>(p[k]);
#pragma unroll
      for (int k = 0; k < 8; ++k) odd[k] = dpp_f<kDppRowShl4>(p[k]);
      if ((xl & 7) == 0) {
        // pair pp = 64 xwv + 8 k + l / 8 of the vector is pair i = pp mod 9 of slice
        // j = pp / 9, whose level-1 index (x, j, i, q) is (288 x + pp) 32 + q
        const int u = __builtin_amdgcn_readfirstlane((x * kPJ * kSliceP + 64 * xwv) * kPJ + c.j);
        const int o = (u + (xl >> 3) * kPJ) * 16;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          u32x4 w;
          w.x = __float_as_uint(p[k]);
          w.y = tag;
          w.z = __float_as_uint(odd[k]);
          w.w = tag;
          __builtin_amdgcn_raw_buffer_store_b128(w, r_p1, o, 8 * kPJ * 16 * k, 0);
        }
      }
      if (xwv == kXW - 1) {
        const float sq = row_sum16(xl < 16 ? ov * ov : 0.f);
        const float dg = row_sum16(xl < 16 ? rc.sg * ov : 0.f);
        if (xl == 0) {
          constexpr int pp = kPartSq / 2, j = pp / kSliceP, i = pp - kSliceP * j;
          u32x4 w;
          w.x = __float_as_uint(sq);
          w.y = tag;
          w.z = __float_as_uint(dg);
          w.w = tag;
          xst2<0>(r_p1, p1_pair(x, j, i, c.j) * 16, w);
        }
      }
    };
    issue_router_cols(rc, a.layer[0], g, xwv, xl);
    publish_part(reinterpret_cast<const float4*>(a.x_in)[4 * g + (xl & 3)], a.x_in[16 * g + (xl & 15)],
                 epoch + 1u, xl);

    for (int L = 0; L < n; ++L) {
      // lane values rebuilt every layer from an opaque copy of the thread index, so that the
      // compiler does not hold loop-invariant addresses across the layer loop
      int tt = c.t;
      asm volatile("" : "+v"(tt));
      const int xl_ = tt & (kWave - 1);
      const PLayer& Ly = a.layer[L];
      const uint32_t tag = epoch + (uint32_t)L + 1u;
      if (xwv == 0) PHASE_STAMP(0);
      // hop 1: slice j over the 32 workgroups of this XCD (lane q of each 32-lane half reads
      // producer q); pairs 2 xwv and 2 xwv + 1 of the slice, and pair 8 in wave 0
      {
        const int i0 = 2 * xwv + (xl_ >> 5), q = xl_ & 31;
        int pr[2] = {p1_pair(x, c.j, i0, q), p1_pair(x, c.j, kSliceP - 1, q)};
        bool act[2] = {kSliceP * c.j + i0 < kPartPairs,
                       xwv == 0 && xl_ < 32 && kSliceP * c.j + kSliceP - 1 < kPartPairs};
        float v[4];
        poll_set<2, 16>(c, r_p1, pr, act, tag, v);
        if (xwv == 0) PHASE_STAMP(1);
        const float s0 = seg_sum<32>(v[0]), s1 = seg_sum<32>(v[1]);
        const float e0 = seg_sum<32>(v[2]), e1 = seg_sum<32>(v[3]);
        if ((xl_ & 31) == 0 && act[0]) {
          u32x4 w;
          w.x = __float_as_uint(s0);
          w.y = tag;
          w.z = __float_as_uint(s1);
          w.w = tag;
          xst2<16>(r_g2, g2_pair(c.j, i0, x) * 16, w);
        }
        if (xwv == 0 && xl_ == 0 && kSliceP * c.j + kSliceP - 1 < kPartPairs) {
          u32x4 w;
          w.x = __float_as_uint(e0);
          w.y = tag;
          w.z = __float_as_uint(e1);
          w.w = tag;
          xst2<16>(r_g2, g2_pair(c.j, kSliceP - 1, x) * 16, w);
        }
      }
      if (xwv <= 1) {
        // hop 2: the 8 XCD partials of slice j, summed in XCD order (every XCD gets the same
        // bits), staged in this XCD's copy; wave 0 takes pairs 0..7 of the slice, wave 1 pair 8
        const int i = xwv == 0 ? (xl_ >> 3) : kSliceP - 1, xp = xl_ & 7;
        int pr[1] = {g2_pair(c.j, i, xp)};
        bool act[1] = {(xwv == 0 || xl_ < 8) && kSliceP * c.j + i < kPartPairs};
        float v[2];
        poll_set<1, 16>(c, r_g2, pr, act, tag, v);
        if (xwv == 0) PHASE_STAMP(2);
        const float s0 = seg_sum<8>(v[0]), s1 = seg_sum<8>(v[1]);
        if (xp == 0 && act[0]) {
          u32x4 w;
          w.x = __float_as_uint(s0);
          w.y = tag;
          w.z = __float_as_uint(s1);
          w.w = tag;
          xst2<0>(r_lpart, (kSliceP * c.j + i) * 16, w);
        }
      }
      if (xwv == 0) {
        // hop 3: the whole reduced vector from this XCD's copy, then the routing
        int pr[5];
        bool act[5];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          pr[m] = xl_ + 64 * m;
          act[m] = true;
        }
        pr[4] = kPartSq / 2;
        act[4] = xl_ == 0;
        float v[10];
        poll_set<5, 16>(c, r_lpart, pr, act, tag, v);
        PHASE_STAMP(3);
        // the top-4 is a dependent chain on this one wave: let it issue ahead of the compute
        // waves that share its SIMD (they only poll the ids flag meanwhile)
        __builtin_amdgcn_s_setprio(3);
        const float sumsq = lane_f(v[8], 0), sgdot = lane_f(v[9], 0);
        float lg[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) lg[m] = v[m];
        int ids[kPK];
        float vals[kPK];
        wave_topk512(lg, xl_, ids, vals);
        // the compute waves need only the ids to start streaming the experts' rows
        if (xl_ < kPK) {
          int id = ids[0];
#pragma unroll
          for (int e = 1; e < kPK; ++e) id = xl_ == e ? ids[e] : id;
          s_ids[xl_] = id;
          if (a.ids_trace && b == 0) a.ids_trace[L * kPK + xl_] = id;
        }
        set_flag((lds_u32*)&flag_ids, tag);
        __builtin_amdgcn_s_setprio(0);
        PHASE_STAMP(4);
        const float s = __builtin_amdgcn_rsqf(sumsq / (float)kPH + a.eps);
        float w[kPK], sum = 0.f;
#pragma unroll
        for (int e = 0; e < kPK; ++e) {
          w[e] = ids[e] >= 0 ? expf((vals[e] - vals[0]) * s) : 0.f;
          sum += w[e];
        }
        const float inv = 1.f / sum;
        if (xl_ < kPK) {
          int id = ids[0];
          float we = w[0];
#pragma unroll
          for (int e = 1; e < kPK; ++e)
            if (xl_ == e) {
              id = ids[e];
              we = w[e];
            }
          s_w[xl_] = (id >= 0 && id < Ly.n_slots) ? we * inv : 0.f;
        }
        if (xl_ == 0) {
          s_scale = s;
          s_sg = sigmoidf_acc(s * sgdot);
        }
        set_flag((lds_u32*)&flag_w, tag);
      } else {
        // the layer input (raw) into xs: wave 2 first moves slice j of the output rows (64
        // pairs) into this XCD's copy; then waves 1..3 read the copy (11 rounds of 192 pairs)
        constexpr int kXsT = (kXW - 1) * kWave, kXsK = (kNOut / 2 + kXsT - 1) / kXsT;
        const int t = tt - kWave;
        float v[2 * kXsK];
        if (L == 0) {
#pragma unroll
          for (int k = 0; k < kXsK; ++k) {
            const int p = t + kXsT * k;
            float2 t2 = make_float2(0.f, 0.f);
            if (p < kNOut / 2) t2 = reinterpret_cast<const float2*>(a.x_in)[p];
            v[2 * k] = t2.x;
            v[2 * k + 1] = t2.y;
          }
        } else {
          if (xwv == 2 && !*(volatile lds_int*)c.abort) {
            const int p = c.j * (kNOut / 2 / kPJ) + xl_;
            const uint64_t t0 = now_ticks();
            u32x4 w0 = xld<16>(r_out, p * 16);
            while (true) {
              const u32x4 w1 = xld<16>(r_out, p * 16);
              if (w0.y == tag && w0.w == tag) {
                xst2<0>(r_lout, p * 16, w0);
                break;
              }
              w0 = xld<16>(r_out, p * 16);
              if (w1.y == tag && w1.w == tag) {
                xst2<0>(r_lout, p * 16, w1);
                break;
              }
              if (*(volatile lds_int*)c.abort) break;
              if (now_ticks() - t0 > kSpinTicks) {
                fail(c, kPersistErrTimeout);
                break;
              }
            }
          }
          int pr[kXsK];
          bool act[kXsK];
#pragma unroll
          for (int k = 0; k < kXsK; ++k) {
            pr[k] = t + kXsT * k;
            act[k] = pr[k] < kNOut / 2;
          }
          // (the input is needed only after the routing: polling it gently leaves the
          // memory system to the routing's all-reduce)
          poll_set<kXsK, 16, 16>(c, r_lout, pr, act, tag, v);
          if (xwv == 2) PHASE_STAMP(15);
        }
        // every exchange wave has read its rows of the previous layer's xs
        if (L > 0) wait_count((lds_u32*)&xread, (uint32_t)kXW * (uint32_t)L);
#pragma unroll
        for (int k = 0; k < kXsK; ++k) {
          const int p = t + kXsT * k;
          if (p < kNOut / 2) {
            xs[2 * p] = v[2 * k];
            xs[2 * p + 1] = v[2 * k + 1];
          }
        }
        add_count((lds_u32*)&flag_x, xl_);
        // the digit planes, once all of xs is in: unit u = 16 inputs 16 u .. 16 u + 15 (chunk
        // u / 2, half u & 1); the four units of a 64-input group sit in one lane quad
        wait_count((lds_u32*)&flag_x, (uint32_t)(kXW - 1) * (uint32_t)(L + 1));
        auto digit_unit = [&](int u) {
          float v[16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 t4 = reinterpret_cast<const float4*>(xs)[4 * u + i];
            v[4 * i] = t4.x;
            v[4 * i + 1] = t4.y;
            v[4 * i + 2] = t4.z;
            v[4 * i + 3] = t4.w;
          }
          // q4 planes: inputs 0..7 and 8..15 of the unit; q2 planes: its even and its odd inputs
          // (the order of the codes that the q2 gate/up product pairs them with)
          uint2 pl[kXPlanes];
          float sum, unit;
          digit_unit16<BITS == 2>(v, pl, sum, unit);
          uint2* dst = reinterpret_cast<uint2*>(xdig[u >> 1]);
#pragma unroll
          for (int k = 0; k < kXPlanes; ++k) dst[2 * k + (u & 1)] = pl[k];
          sum += dpp_f<kDppQuadXor1>(sum);
          if ((u & 1) == 0) xaux[u >> 1] = make_float2(sum, unit);
        };
        digit_unit(kWave * (xwv - 1) + xl_);
        if (xwv == 1) digit_unit(kWave * (kXW - 1) + xl_);
        add_count((lds_u32*)&flag_xd, xl_);
        if (xwv == 2) PHASE_STAMP(16);
      }
      // the 80 down rows: exchange wave v loads pairs 20 v .. 20 v + 19, kRPI rows per
      // instruction (2 for q4, 4 for q2: 16 bytes per lane), and their scale/bias (lane l of
      // step m: chunk 64 m + l -> row chunk / 4, segment (chunk / 2) & 1, part chunk & 1),
      // queued behind the compute waves' gate/up rows
      constexpr int kRPI = kWave / P::kDnU4, kNI = 20 / kRPI;
      v4u dnr[kNI], dmr[2];
      {
        wait_count((lds_u32*)&gu_issued, (uint32_t)kCW * (uint32_t)(L + 1));
        const uint8_t* dsl[kPS];
#pragma unroll
        for (int e = 0; e < kPK; ++e) {
          const int id = __builtin_amdgcn_readfirstlane(s_ids[e]);
          dsl[e] = Ly.base + (size_t)(id >= 0 && id < Ly.n_slots ? id : 0) * Ly.slot_bytes;
        }
        dsl[kPK] = Ly.base + (size_t)Ly.shared_slot * Ly.slot_bytes;
        auto slot_of = [&](int p) {
          const int e = p >> 4;
          return e == 0 ? dsl[0] : e == 1 ? dsl[1] : e == 2 ? dsl[2] : e == 3 ? dsl[3] : dsl[4];
        };
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int ch = 64 * m + xl_ < 80 ? 64 * m + xl_ : xl_;
          const int p = 20 * xwv + (ch >> 2);
          dmr[m] = ld_nt_ptr(
              dn_meta_addr<BITS>(slot_of(p), 16 * g + (p & 15), (ch >> 1) & 1, ch & 1));
        }
#pragma unroll
        for (int k = 0; k < kNI; ++k) {
          const int p = 20 * xwv + kRPI * k + xl_ / P::kDnU4;
          dnr[k] = ld_nt_ptr(slot_of(p) + P::kDnOff + (size_t)(16 * g + (p & 15)) * P::kDnRow +
                             (xl_ % P::kDnU4) * 16);
        }
      }
      if (xwv == 0) PHASE_STAMP(9);
      // park the down rows in LDS (this wave's exchange loads below return after them anyway)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int ch = 64 * m + xl_;
        if (ch < 80) dn_meta[20 * xwv + (ch >> 2)][((ch >> 1) & 1) * 2 + (ch & 1)] =
            make_uint4(dmr[m][0], dmr[m][1], dmr[m][2], dmr[m][3]);
      }
#pragma unroll
      for (int k = 0; k < kNI; ++k)
        dn_codes[20 * xwv + kRPI * k + xl_ / P::kDnU4][xl_ % P::kDnU4] =
            make_uint4(dnr[k][0], dnr[k][1], dnr[k][2], dnr[k][3]);
      add_count((lds_u32*)&dn_parked, xl_);  // the compute waves pre-convert their rows' codes
      {
        // straight from the global buffer: one cross-XCD round trip after the last producer,
        // where fetching slices into a per-XCD copy first costs a second one
        if constexpr (BITS == 4) {
          float v[kNH / kXT];
          poll_pairs<kNH / 2 / kXT, kNH / 2, kXT, 16>(c, tt, rsrc(reinterpret_cast<uint8_t*>(xw.g_h) + (size_t)(x % kHCopies<BITS>) * PersistWs::kGHCopy), tag, v);
#pragma unroll
          for (int i = 0; i < kNH / kXT / 2; ++i) {
            const int p = tt + kXT * i;
            hs[2 * p] = v[2 * i];
            hs[2 * p + 1] = v[2 * i + 1];
          }
        } else {
          float4 v[kNH / 4 / kXT];
          poll_h<kNH / 4 / kXT>(c, tt, rsrc(reinterpret_cast<uint8_t*>(xw.g_h) + (size_t)(x % kHCopies<BITS>) * PersistWs::kGHCopy), tag, v);
#pragma unroll
          for (int i = 0; i < kNH / 4 / kXT; ++i)
            reinterpret_cast<float4*>(hs)[tt + kXT * i] = v[i];
        }
      }
      if (xwv == 0) PHASE_STAMP(10);
      wg_barrier();  // E
      if (xwv == 0) PHASE_STAMP(11);
      // the next layer's router columns: the first loads after barrier E, so that they have
      // landed by this layer's publish (issued before E they would slow the last SwiGLU polls of
      // the other exchange waves)
      if (L + 1 < n) issue_router_cols(rc, a.layer[L + 1], g, xwv, xl_);
      // the shared slot's rows at a raised issue priority: the exchange wave is the third on its
      // SIMD and would otherwise get the VALU only after both compute waves are done
      __builtin_amdgcn_s_setprio(2);
      {
        // the shared slot's down rows 4 xwv .. 4 xwv + 3
        float y[4];
        down_partials<BITS, 4>(hs, dn_codes, dn_meta, kPK * 16 + 4 * xwv, xl_, y);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = seg_sum<kWave>(y[i]);
          if (xl_ == 0) ydn[kPK][4 * xwv + i] = v;
        }
      }
      __builtin_amdgcn_s_setprio(0);
      wg_barrier();  // F
      if (xwv == 0) PHASE_STAMP(13);
      // this workgroup's 16 output rows: to the other workgroups (the next layer's input, or
      // the stack output), and as the next layer's partial router sums.  On the last layer
      // only wave 0 reads xs here: the final gather below rewrites it.
      if (xwv == 0 || L + 1 < n) {
        const float v = out_row(xl_ & 15);
        if (xwv == 0 && xl_ < 16) {
          const int row = 16 * g + xl_;
          xst1(r_out, row, v, tag + 1u);
          if (L == n - 1) a.x_out[row] = v;
        }
        if (L + 1 < n) {
          const int c4 = 4 * (xl_ & 3);
          const float4 ow = make_float4(out_row(c4), out_row(c4 + 1), out_row(c4 + 2), out_row(c4 + 3));
          add_count((lds_u32*)&xread, xl_);
          publish_part(ow, v, tag + 1u, xl_);
          if (xwv == 0) PHASE_STAMP(14);
        }
      }
    }
    // RMSNorm of the stack output (every workgroup needs the full sum of squares)
    const uint32_t tag = epoch + (uint32_t)n + 1u;
    {
      float v[kNOut / kXT];
      gather<kNOut, kXT>(c, c.t, xw.g_out, xw.l_out, tag, v);
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < kNOut / kXT / 2; ++i) {
        const int p = c.t + kXT * i;
        xs[2 * p] = v[2 * i];
        xs[2 * p + 1] = v[2 * i + 1];
        sq = fmaf(v[2 * i], v[2 * i], sq);
        sq = fmaf(v[2 * i + 1], v[2 * i + 1], sq);
      }
      sq = seg_sum<kWave>(sq);
      if (xl == 0) xsq[xwv] = sq;
    }
    x_barrier(c, bar, xgen);
    if (a.xn_out && c.t < 16) {
      const float ss = (xsq[0] + xsq[1]) + (xsq[2] + xsq[3]);
      const float sn = __builtin_amdgcn_rsqf(ss / (float)kPH + a.eps);
      const int row = 16 * g + c.t;
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

#ifdef MOE_PHASE_STAMPS
uint64_t* g_stamps = nullptr;  // the instrumentation build's stamp buffer (null: no stamps)
#endif

bool persist_shape_ok(const moe_layer* layers, int n_layers) {
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    if (L.experts.bits != layers[0].experts.bits ||
        (L.experts.bits != 4 && L.experts.bits != 2) || L.experts.hidden != kPH ||
        L.experts.inter != kPI ||
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
                          bool plain_launch, hipStream_t stream) {
  PArgs a{};
  a.n_layers = n_layers;
  a.eps = eps;
  a.x_in = x_in;
  a.x_out = x_out;
  a.xn_out = xn_out;
  a.ids_trace = ids_trace;
  a.xw = xw_base;
  a.dev_err = layers[0].experts.dev_err;
#ifdef MOE_PHASE_STAMPS
  a.stamps = g_stamps;
#endif
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    a.layer[l].base = reinterpret_cast<const uint8_t*>(L.experts.base);
    a.layer[l].w_router = L.w_router;
    a.layer[l].w_router_cb = L.w_router_cb;
    a.layer[l].w_sg = L.w_sg;
    a.layer[l].slot_bytes = L.experts.slot_bytes;
    a.layer[l].n_slots = L.experts.n_slots;
    a.layer[l].shared_slot = L.shared_slot;
  }
  // A cooperative launch guarantees that all 256 workgroups are resident at once.  Tracing
  // tools that cannot follow cooperative launches get the same kernel through an ordinary
  // launch (plain_launch): on an otherwise idle device the 256 workgroups (one per CU) are
  // still all resident; if they are not, the bounded waits report a timeout through dev_err
  // instead of hanging.
  const void* kern = layers[0].experts.bits == 4
                         ? reinterpret_cast<const void*>(persist_kernel<4>)
                         : reinterpret_cast<const void*>(persist_kernel<2>);
  if (plain_launch) {
    if (layers[0].experts.bits == 4)
      hipLaunchKernelGGL(persist_kernel<4>, dim3(kPB), dim3(kPT), 0, stream, a);
    else
      hipLaunchKernelGGL(persist_kernel<2>, dim3(kPB), dim3(kPT), 0, stream, a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
  }
  void* args[] = {&a};
  const hipError_t e = hipLaunchCooperativeKernel(kern, dim3(kPB), dim3(kPT), args, 0, stream);
  return e == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // namespace moe

#ifdef MOE_PHASE_STAMPS
// Instrumentation build only: every later persistent launch writes its phase stamps to buf, a
// device buffer of at least kPersistMaxLayers x 256 x 32 uint64 (NULL turns the stamps off).
extern "C" void moe_phase_stamps(void* buf) { moe::g_stamps = static_cast<uint64_t*>(buf); }
#endif
