// Weight-streaming grouped GEMMs on bf16 (or fp32) MFMA: the SwiGLU expert
// FFN (gate/up with a fused SiLU-multiply, down with the router-weight scale
// and the scatter to the token's slot) and the LM head with a blocked arg max.
//
// Experts: "The speed comes from three layers working together" (Jina-OCR-v1
// explainer, kg.zhiyong.dev) -- 64 routed and two always-on shared experts,
// top-6 routing.  Greedy head: "Why FastMTP fits OCR particularly well" (same
// page) -- verification reproduces greedy decoding, so the head's output is an
// arg max with a fixed tie rule (lowest vocabulary index).
//
// Design (decode shapes are weight-bandwidth bound: every expert's weights
// are read from HBM exactly once per call):
//   * weights are stored fragment-packed: for each tile of 16 rows and each
//     32-wide K block, the 64 lanes' 16-byte A fragments lie contiguously
//     (1 KB for bf16), and consecutive K blocks of a tile are adjacent, so a
//     wavefront streams one contiguous region with full-line loads;
//   * one workgroup = 4 wavefronts owns a slab of 64 (or 64*RT) weight rows of
//     one group and ALL of that group's tokens (in passes), so no weight byte
//     is fetched twice; each wavefront owns RT tiles of 16 rows;
//   * A fragments go straight from HBM into a register ring several K blocks
//     deep, so requests for later blocks are in flight while the current one
//     is multiplied;
//   * passes of at most 32 tokens (the routed experts at decode batch sizes)
//     fetch their token fragments straight from global memory (L2) through
//     the same ring -- no LDS, no barriers; larger passes stage the token rows
//     through LDS in 64-wide K chunks shared by the 4 wavefronts (rows padded
//     by 16 bytes so the 16-byte fragment reads of 16 rows hit distinct banks);
//   * every output element is a single fp32 accumulation over K in the same
//     block order whatever path or pass size ran it, so a token's result does
//     not depend on its batch companions.
#include "launch.h"

namespace moev {
namespace {

enum Mode { kGateUp = 0, kDown = 1, kHead = 2 };

constexpr int kKC = 64;              // K elements per LDS chunk (multiple of 32)
constexpr int kKB = kKC / 32;        // MFMA K blocks per chunk
constexpr int kNB = 3;               // LDS path: weight ring depth in chunks
constexpr int kNBD = 4;              // direct path: ring depth in K blocks
constexpr int kFrag = 512;           // elements of one packed 16x32 fragment
constexpr int kRtDown = 1;           // 16-row tiles per wave, down projection
constexpr int kRtHead = 2;           // 16-row tiles per wave, LM head
constexpr int kWavesFfn = 4;         // wavefronts per workgroup, expert GEMMs
constexpr int kTileMinTokens = 128;  // larger batches use the tile schedule
constexpr int kWavesHead = 8;        // wavefronts per workgroup, LM head
static_assert(kTileMinTokens <= 128 && kSetMaxTokens <= 512,
              "token sets: two mask words on the streaming schedule, at most eight on the tiled one");

// MT = tokens per pass (32, 64 or 128 = 2, 4 or 8 MFMA column tiles).  The
// variant only changes how many accumulators and LDS rows a workgroup holds;
// every variant adds the same K blocks in the same order, so a token's result
// is the same bits whichever variant ran it.
template <typename WT, int MT> struct Cfg {
  static constexpr int kEpv = 16 / sizeof(WT);                     // elements per 16 B
  static constexpr int kRowBytes = kKC * sizeof(WT) + 16;          // padded LDS row
  static constexpr int kVecPerRow = kKC * sizeof(WT) / 16;         // 16-B vectors per row
  static constexpr int kTiles = MT / 16;                           // MFMA column tiles
  static constexpr int kRedBytes = 8 * kWavesHead * MT;            // head arg max scratch
  static constexpr int kLdsBytes = MT * kRowBytes > kRedBytes ? MT * kRowBytes : kRedBytes;
};

struct GemmArgs {
  const void* w0;           // packed [G][N/16][K/32][512] (gate/up: gate; down; head)
  const void* w1;           // gate/up: up, else unused
  long long w_group;        // elements between consecutive groups
  int N, K;                 // weight rows per group, contraction length
  const void* x;            // operand rows
  const int32_t* offsets;   // [G+1] (gate/up, down)
  const int32_t* sorted_src;
  // token-set mode: routed group g < E holds the tokens whose bit is set in
  // its mask words (masks[set_word(E, g, w)]), shared groups every
  // token; group g's m-th token has act row g*T + m (see TokenSets)
  bool sets;
  int E, W;
  const uint64_t* masks;    // [W][E]
  const int2* pinfo;        // [T][E] (down): {bits of the pair's weight, slot}

  int S, k, P, T;           // slots, routed slots, pairs, tokens
  int n_first;              // the last n_first groups (the shared experts, which
                            // hold every token) are dispatched first
  const float* topk_w;      // [T, k] (down)
  void* out;                // gate/up: act [P, N] WT; down: y [P, N] fp32; head: pmax
  int32_t* out_idx;         // head: partial arg max [T, blocks]
  float* logits;            // head: optional logits [T, N]
  QkvScatter scatter;       // down: where a fused Q/K/V projection's rows go
  bool scattered;           //   (instead of out) when set
};

// SwiGLU combination silu(g) * u = g / (1 + e^-g) * u from the hardware
// base-2 exponential (v_exp_f32) and reciprocal (v_rcp_f32), each within
// about one ulp; every GEMM schedule uses this one expression, so the
// schedules agree bit for bit.  Large negative g: e^-g overflows to inf and
// the product is -0; large positive g: e^-g underflows to 0 and the result
// is g * u.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

template <typename WT> __device__ __forceinline__ void store4(WT* p, f32x4 v);
template <> __device__ __forceinline__ void store4<u16>(u16* p, f32x4 v) {
  uint2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

// Position of the m-th set bit (m counted from 0) of the 128-bit set
// {lo, hi}; m is below the set's population count.  Halving search on the
// population counts of the lower halves.
__device__ __forceinline__ int nth_set_bit(uint64_t lo, uint64_t hi, int m) {
  const int c = __popcll(lo);
  uint64_t w = m < c ? lo : hi;
  int pos = m < c ? 0 : 64;
  m = m < c ? m : m - c;
#pragma unroll
  for (int sh = 32; sh > 0; sh >>= 1) {
    const int cl = __popcll(w & ((1ull << sh) - 1));
    if (m >= cl) {
      m -= cl;
      w >>= sh;
      pos += sh;
    }
  }
  return pos;
}

// The tokens of one group of the token-set mode: a routed group's mask, or
// every token (masked = false).
struct TokenSel {
  uint64_t lo = 0, hi = 0;
  bool masked = false;
  int g = 0;
};

__device__ __forceinline__ int set_token(const GemmArgs& a, const TokenSel& sel, int m) {
  return sel.masked ? min(nth_set_bit(sel.lo, sel.hi, m), a.T - 1) : m;
}

// Token sets on the tiled schedule (up to eight mask words): the size of
// routed group g's set, and its m-th token (clamped to a row).  Both load
// every word up front (clamped to the last one, so all loads are in bounds and
// independent) and then count in registers.
constexpr int kSetMaxWords = kSetMaxTokens / 64;
__device__ __forceinline__ void set_load(const GemmArgs& a, int g, uint64_t (&x)[kSetMaxWords]) {
#pragma unroll
  for (int w = 0; w < kSetMaxWords; ++w) x[w] = a.masks[set_word(a.E, g, min(w, a.W - 1))];
}
__device__ __forceinline__ int set_size(const GemmArgs& a, int g) {
  uint64_t x[kSetMaxWords];
  set_load(a, g, x);
  int n = 0;
#pragma unroll
  for (int w = 0; w < kSetMaxWords; ++w) n += w < a.W ? __popcll(x[w]) : 0;
  return min(n, a.T);
}
__device__ __forceinline__ int set_nth(const GemmArgs& a, int g, int m) {
  uint64_t x[kSetMaxWords];
  set_load(a, g, x);
  int base = 0;
#pragma unroll
  for (int w = 0; w < kSetMaxWords; ++w) {
    if (w >= a.W) break;
    const int c = __popcll(x[w]);
    if (m < c) return min(base + nth_set_bit(x[w], 0ull, m), a.T - 1);
    m -= c;
    base += 64;
  }
  return a.T - 1;
}

// Four gain elements as loaded (bf16 pairs or fp32), converted when used.
template <typename WT> struct GainRaw;
template <> struct GainRaw<u16> {
  using T = uint2;
  __device__ static uint2 load(const u16* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ static float4 to_f4(uint2 u) {
    return make_float4(bf16_to_f32(u.x & 0xFFFF), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xFFFF),
                       bf16_to_f32(u.y >> 16));
  }
};
template <> struct GainRaw<float> {
  using T = float4;
  __device__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static float4 to_f4(float4 v) { return v; }
};

// Row of the operand matrix that token row `row` of this pass reads.  SETS =
// false (the tile schedule, which never runs on token sets) compiles the
// sorted-order read only.
template <int MODE, bool SETS = true>
__device__ __forceinline__ long long operand_row(const GemmArgs& a, const TokenSel& sel, int off, int m0,
                                                 int row) {
  if (MODE == kGateUp)
    return (SETS && a.sets) ? set_token(a, sel, m0 + row)
                            : clampi(a.sorted_src[off + m0 + row], 0, a.P - 1) / a.S;
  if (MODE == kDown) return off + m0 + row;
  return m0 + row;
}

// Operand row of token row `row` of a tile pass (the tiled schedule): with
// token sets a gate/up tile of routed group g reads its m-th token's row.
template <int MODE, bool SETS>
__device__ __forceinline__ long long tile_row(const GemmArgs& a, int g, int off, int m0, int row) {
  if constexpr (SETS && MODE == kGateUp) return g < a.E ? set_nth(a, g, m0 + row) : m0 + row;
  else return operand_row<MODE, false>(a, TokenSel{}, off, m0, row);
}

// Down projection: output pair and router weight of token row m of a pass,
// read when the pass starts so the epilogue does not wait for them.
struct PairMeta {
  int p = 0;
  float wgt = 1.f;
};

__device__ __forceinline__ PairMeta pair_meta(const GemmArgs& a, const TokenSel& sel, int off, int m) {
  PairMeta r;
  int t, slot;
  if (a.sets) {
    t = set_token(a, sel, m);
    if (sel.masked) {
      const int2 pi = a.pinfo[static_cast<long long>(t) * a.E + sel.g];
      slot = clampi(pi.y, 0, a.k - 1);
      r.wgt = __int_as_float(pi.x);
    } else {
      slot = a.k + sel.g - a.E;
    }
    r.p = t * a.S + slot;
  } else {
    r.p = clampi(a.sorted_src[off + m], 0, a.P - 1);
    t = r.p / a.S;
    slot = r.p - t * a.S;
    if (slot < a.k) r.wgt = a.topk_w[static_cast<long long>(t) * a.k + slot];
  }
  return r;
}

template <int MODE, int NTX>
__device__ __forceinline__ void load_meta(const GemmArgs& a, const TokenSel& sel, int off, int m0, int mp,
                                          PairMeta (&meta)[NTX]) {
  if constexpr (MODE == kDown) {
    const int r16 = threadIdx.x & 15;
#pragma unroll
    for (int j = 0; j < NTX; ++j) {
      const int m = j * 16 + r16;
      if (m < mp) meta[j] = pair_meta(a, sel, off, m0 + m);
    }
  }
}

// Four adjacent output columns col.. of row t of a fused Q/K/V projection
// (N = 3H): q columns to the fp32 q rows, key and value columns to the
// caches at the row's position, rounded like every other cache write.  The
// four columns share one head (D and H are multiples of 4).
template <typename WT>
__device__ __forceinline__ void qkv_store(const GemmArgs& a, int t, int col, f32x4 o) {
  const QkvScatter& sc = a.scatter;
  const int H = a.N / 3;
  const int b = t / sc.rows, i = t - b * sc.rows;
  const int p0 = sc.pos[b];
  if (p0 < 0 || p0 > sc.max_len - sc.rows) return;
  if (col < H) {
    store4<float>(sc.q + static_cast<long long>(t) * H + col, o);
    return;
  }
  const bool key = col < 2 * H;
  const int c = col - (key ? H : 2 * H);
  const int sh = __ffs(sc.D) - 1;  // D is a power of two
  const int hd = c >> sh, d = c & (sc.D - 1);
  const long long dst = ((static_cast<long long>(b) * (H >> sh) + hd) * sc.max_len + p0 + i) * sc.D + d;
  store4<WT>(static_cast<WT*>(key ? sc.k_cache : sc.v_cache) + dst, o);
}

// Epilogue of one pass: lane (r16, q) holds rows rowbase[rt] + 4q + v of
// token column j*16 + r16.
// SCATTER: the build may write a fused Q/K/V projection's rows (split-K
// dense projections only; the expert GEMMs never do).
template <typename WT, int MODE, int RT, int MT, int NTX, int W, bool SCATTER = false>
__device__ __forceinline__ void epilogue(const GemmArgs& a, unsigned char* __restrict__ lds,
                                         const f32x4 (&acc)[RT][NTX], int off, int m0, int mp,
                                         const int (&rowbase)[RT], const PairMeta (&meta)[NTX]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int mt = (mp + 15) >> 4;
  if (MODE == kGateUp) {
    WT* act = static_cast<WT*>(a.out);
    const int n = rowbase[0] + 4 * q;
#pragma unroll
    for (int j = 0; j < NTX; ++j) {
      const int m = j * 16 + r16;
      if (m < mp) {
        f32x4 gv = acc[0][j], uv = acc[1][j], o;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = silu_mul(gv[v], uv[v]);
        store4<WT>(act + static_cast<long long>(off + m0 + m) * a.N + n, o);
      }
    }
  } else if (MODE == kDown) {
    float* y = static_cast<float*>(a.out);
#pragma unroll
    for (int j = 0; j < NTX; ++j) {
      const int m = j * 16 + r16;
      if (m < mp) {
        const int p = meta[j].p;
        const float wgt = meta[j].wgt;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          f32x4 o = acc[rt][j];
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] *= wgt;
          if (SCATTER && a.scattered) qkv_store<WT>(a, p, rowbase[rt] + 4 * q, o);
          else store4<float>(y + static_cast<long long>(p) * a.N + rowbase[rt] + 4 * q, o);
        }
      }
    }
  } else {
    // per token column: best (value, vocab index) over this wave's rows
    __syncthreads();  // every wave is done with the staged chunk
    float* red_v = reinterpret_cast<float*>(lds);         // [W][MT]
    int* red_i = reinterpret_cast<int*>(lds) + W * MT;    // [W][MT]
#pragma unroll
    for (int j = 0; j < NTX; ++j) {
      if (j < mt) {
        const int m = j * 16 + r16;
        float best = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = rowbase[rt] + 4 * q + v;
            if (n < a.N) {
              const float val = acc[rt][j][v];
              if (a.logits != nullptr && m < mp) a.logits[static_cast<long long>(m0 + m) * a.N + n] = val;
              if (better(val, n, best, bi)) { best = val; bi = n; }
            }
          }
#pragma unroll
        for (int msk = 16; msk <= 32; msk <<= 1) {
          const float ov = __shfl_xor(best, msk, kWave);
          const int oi = __shfl_xor(bi, msk, kWave);
          if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
        }
        if (q == 0) {
          red_v[wave * MT + m] = best;
          red_i[wave * MT + m] = bi;
        }
      }
    }
    __syncthreads();
    if (tid < mp) {
      float best = red_v[tid];
      int bi = red_i[tid];
#pragma unroll
      for (int w = 1; w < W; ++w) {
        const float ov = red_v[w * MT + tid];
        const int oi = red_i[w * MT + tid];
        if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
      }
      const long long o = static_cast<long long>(m0 + tid) * gridDim.x + blockIdx.x;  // [T][blocks]
      static_cast<float*>(a.out)[o] = best;
      a.out_idx[o] = bi;
    }
  }
}

// Direct pass (mp <= 16 * NTX <= 32): both fragments come from global memory
// through one register ring kNBD K blocks deep; no LDS, no barriers.  Token
// rows past mp read row 0 of the pass and are dropped by the epilogue.
//
// KS > 1 (split K): the workgroup's KS = W waves share one row tile, wave w
// takes K blocks [w*nkb/KS, (w+1)*nkb/KS) in order, and wave 0 adds the
// other waves' partial sums (w = 1, 2, ... in turn, through LDS) before its
// epilogue.  The sum order is fixed, so a token's result does not depend on
// its pass companions; it differs in rounding from the single-chain order
// of KS = 1, so a caller uses one KS for all its sizes.
template <typename WT, int MODE, int RT, int MT, int NTX, int W, int KS = 1>
__device__ __forceinline__ void gemm_pass_direct(const GemmArgs& a, unsigned char* __restrict__ lds,
                                                 const TokenSel& sel, int off, int m0, int mp,
                                                 const WT* const (&wp)[RT],
                                                 const int (&rowbase)[RT]) {
  static_assert(KS == 1 || (KS == W && MODE != kHead), "split K: one K range per wave, expert GEMMs");
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int K = a.K;
  const int wave = threadIdx.x >> 6;
  const int kb_lo = KS > 1 ? wave * (K / 32) / KS : 0;
  const int nkb = KS > 1 ? (wave + 1) * (K / 32) / KS : K / 32;  // end of this wave's range
  const WT* __restrict__ xsrc = static_cast<const WT*>(a.x);
  const WT* xp[NTX];
#pragma unroll
  for (int j = 0; j < NTX; ++j) {
    const int m = j * 16 + r16;
    xp[j] = xsrc + operand_row<MODE>(a, sel, off, m0, m < mp ? m : 0) * K + q * 8;
  }
  PairMeta meta[NTX];
  load_meta<MODE, NTX>(a, sel, off, m0, mp, meta);
  f32x4 acc[RT][NTX];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NTX; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // bf16 down projection: the steady-state loop below (the prologue then
  // loads every slot, clamped to the range)
  constexpr bool kSteady = sizeof(WT) == 2 && MODE == kDown;
  Frag<WT> rw[kNBD][RT], rx[kNBD][NTX];
#pragma unroll
  for (int u = 0; u < kNBD; ++u)
    if (kSteady || kb_lo + u < nkb) {
      const int kb = min(kb_lo + u, nkb - 1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) rw[u][rt].load(wp[rt] + kb * kFrag);
#pragma unroll
      for (int j = 0; j < NTX; ++j) rx[u][j].load(xp[j] + kb * 32);
    }
  // the K loop as a ring of kNBD slots, loads skipped past the range
  auto ring_loop = [&]() __attribute__((always_inline)) {
  for (int kb0 = kb_lo; kb0 < nkb; kb0 += kNBD) {
#pragma unroll
    for (int u = 0; u < kNBD; ++u) {
      const int kb = kb0 + u;
      if (kb < nkb) {
#pragma unroll
        for (int j = 0; j < NTX; ++j)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt][j] = mma(rw[u][rt], rx[u][j], acc[rt][j]);
        if (kb + kNBD < nkb) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) rw[u][rt].load(wp[rt] + (kb + kNBD) * kFrag);
#pragma unroll
          for (int j = 0; j < NTX; ++j) rx[u][j].load(xp[j] + (kb + kNBD) * 32);
        }
      }
    }
  }
  };
  if constexpr (kSteady) {
    if ((nkb - kb_lo) % kNBD == 0) {
      // Steady state: every round loads all of the next round's slots (all
      // in range), so each wait covers one slot, and the last round loads
      // nothing.  (The ring loop's skipped loads make the count of loads in
      // flight path-dependent, and the compiler then drains the ring at the
      // top of every round; for gate/up that drained loop measured faster,
      // and this one does not fit its registers at two waves per SIMD.)
      int kb0 = kb_lo;
      for (; kb0 + kNBD < nkb; kb0 += kNBD) {
#pragma unroll
        for (int u = 0; u < kNBD; ++u) {
#pragma unroll
          for (int j = 0; j < NTX; ++j)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[rt][j] = mma(rw[u][rt], rx[u][j], acc[rt][j]);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) rw[u][rt].load(wp[rt] + (kb0 + u + kNBD) * kFrag);
#pragma unroll
          for (int j = 0; j < NTX; ++j) rx[u][j].load(xp[j] + (kb0 + u + kNBD) * 32);
          // each slot's loads right after its MFMAs (the scheduler would
          // otherwise sink a round's loads to its end)
          __builtin_amdgcn_sched_group_barrier(0x008, RT * NTX, 0);  // MFMAs
          __builtin_amdgcn_sched_group_barrier(0x020, RT + NTX, 0);  // vector memory reads
        }
      }
#pragma unroll
      for (int u = 0; u < kNBD; ++u)
#pragma unroll
        for (int j = 0; j < NTX; ++j)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt][j] = mma(rw[u][rt], rx[u][j], acc[rt][j]);
    } else {
      ring_loop();
    }
  } else {
    ring_loop();
  }
  if constexpr (KS > 1) {
    __shared__ f32x4 red[KS - 1][RT][NTX][kWave];
    if (wave > 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int j = 0; j < NTX; ++j) red[wave - 1][rt][j][lane] = acc[rt][j];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < KS - 1; ++w)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int j = 0; j < NTX; ++j) {
            const f32x4 o = red[w][rt][j][lane];
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[rt][j][v] += o[v];
          }
      epilogue<WT, MODE, RT, MT, NTX, W, true>(a, lds, acc, off, m0, mp, rowbase, meta);
    }
    __syncthreads();  // red is free for the next pass
  } else {
    epilogue<WT, MODE, RT, MT, NTX, W>(a, lds, acc, off, m0, mp, rowbase, meta);
  }
}

// LDS-staged pass: mt = ceil(mp / 16) <= NTX column tiles.  NTX is a
// compile-time tile count, so the K loop carries no per-tile predicates;
// tiles past mt multiply LDS rows that the staging loop zero-filled and are
// dropped by the epilogue.
template <typename WT, int MODE, int RT, int MT, int NTX, int W>
__device__ __forceinline__ void gemm_pass_lds(const GemmArgs& a, unsigned char* __restrict__ lds,
                                              const TokenSel& sel, int off, int m0, int mp,
                                              const WT* const (&wp)[RT], const int (&rowbase)[RT]) {
  using C = Cfg<WT, MT>;
  constexpr int kThreads = W * kWave;
  constexpr int kVecs = 16 * NTX * C::kVecPerRow;                // 16-B vectors per chunk
  constexpr int kStage = (kVecs + kThreads - 1) / kThreads;      // staging vectors per thread
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int K = a.K;
  const int nchunks = K / kKC;
  const WT* __restrict__ xsrc = static_cast<const WT*>(a.x);

  // source rows for this thread's staging vectors (nullptr: zero-fill)
  const WT* src[kStage];
#pragma unroll
  for (int s = 0; s < kStage; ++s) {
    const int v = tid + s * kThreads;
    const int row = v / C::kVecPerRow;
    const int cv = v - row * C::kVecPerRow;
    src[s] = (v < kVecs && row < mp) ? xsrc + operand_row<MODE>(a, sel, off, m0, row) * K + cv * C::kEpv
                                     : nullptr;
  }
  PairMeta meta[NTX];
  load_meta<MODE, NTX>(a, sel, off, m0, mp, meta);
  uint4 stage[kStage];
#pragma unroll
  for (int s = 0; s < kStage; ++s)
    stage[s] = src[s] ? *reinterpret_cast<const uint4*>(src[s]) : make_uint4(0, 0, 0, 0);

  f32x4 acc[RT][NTX];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NTX; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Ring loads skipped past the last chunk make the number of loads in flight
  // depend on the path, and the compiler then waits for all of them at the
  // top of every ring round.  The down projection loads every slot instead
  // (clamped to the last chunk), so its waits cover one slot's loads; for
  // gate/up that measured slower at uniform routing, so it keeps the skips.
  constexpr bool kAllLoads = MODE == kDown;
  const int last = nchunks - 1;
  Frag<WT> ring[kNB][RT][kKB];
#pragma unroll
  for (int u = 0; u < kNB; ++u)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int kk = 0; kk < kKB; ++kk)
        if (kAllLoads || u < nchunks) ring[u][rt][kk].load(wp[rt] + (min(u, last) * kKB + kk) * kFrag);

  for (int c0 = 0; c0 < nchunks; c0 += kNB) {
#pragma unroll
    for (int u = 0; u < kNB; ++u) {
      const int c = c0 + u;
      if (c < nchunks) {
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kStage; ++s) {
          const int v = tid + s * kThreads;
          const int row = v / C::kVecPerRow;
          const int cv = v - row * C::kVecPerRow;
          if (v < kVecs) *reinterpret_cast<uint4*>(lds + row * C::kRowBytes + cv * 16) = stage[s];
        }
        __syncthreads();
        if (c + 1 < nchunks) {
#pragma unroll
          for (int s = 0; s < kStage; ++s)
            if (src[s]) stage[s] = *reinterpret_cast<const uint4*>(src[s] + (c + 1) * kKC);
        }
#pragma unroll
        for (int kk = 0; kk < kKB; ++kk) {
#pragma unroll
          for (int j = 0; j < NTX; ++j) {
            Frag<WT> b;
            b.load(reinterpret_cast<const WT*>(lds + (j * 16 + r16) * C::kRowBytes) + kk * 32 + q * 8);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[rt][j] = mma(ring[u][rt][kk], b, acc[rt][j]);
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int kk = 0; kk < kKB; ++kk)
            if (kAllLoads || c + kNB < nchunks)
              ring[u][rt][kk].load(wp[rt] + (min(c + kNB, last) * kKB + kk) * kFrag);
      }
    }
  }
  epilogue<WT, MODE, RT, MT, NTX, W>(a, lds, acc, off, m0, mp, rowbase, meta);
}

// One workgroup of the streaming schedule: row slab bx of group slot by,
// token passes bz, bz + nz, ...  (G groups; the last a.n_first are
// dispatched first).
template <typename WT, int MODE, int RT, int MT, int W, int KS = 1>
__device__ __forceinline__ void stream_gemm_wg(const GemmArgs& a, int bx, int by, int bz, int G, int nz) {
  static_assert(KS == 1 || MT == 32, "split K runs direct passes of at most 32 tokens");
  using C = Cfg<WT, MT>;
  constexpr int NT = C::kTiles;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  int g = 0, off = 0, M;
  TokenSel sel;
  if (MODE == kHead) {
    M = a.T;
  } else {
    g = by < a.n_first ? G - a.n_first + by : by - a.n_first;
    sel.g = g;
    if (a.sets) {
      off = g * a.T;
      M = a.T;
      if (g < a.E) {
        sel.lo = a.masks[set_word(a.E, g, 0)];
        sel.hi = a.W > 1 ? a.masks[set_word(a.E, g, 1)] : 0ull;
        sel.masked = true;
        M = min(__popcll(sel.lo) + __popcll(sel.hi), a.T);
      }
    } else {
      off = clampi(a.offsets[g], 0, a.P);
      M = clampi(a.offsets[g + 1], off, a.P) - off;
    }
  }
  if (M <= 0) return;

  const WT* __restrict__ w0 = static_cast<const WT*>(a.w0);
  const WT* __restrict__ w1 = static_cast<const WT*>(a.w1);
  const int nkb = a.K / 32;
  const int ntiles = (a.N + 15) / 16;

  // this wave's weight tiles; lane pointer = its 16 bytes of the first fragment
  // (split K: every wave of the workgroup has the same tiles)
  const WT* wp[RT];
  int rowbase[RT];
  constexpr int kWaveTiles = KS > 1 ? 1 : W;  // row tiles (of 16 x RT rows) per workgroup
  const int wt = KS > 1 ? 0 : wave;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rb = (MODE == kGateUp) ? bx * (16 * kWaveTiles) + wt * 16
                                     : bx * (16 * RT * kWaveTiles) + wt * (16 * RT) + rt * 16;
    rowbase[rt] = rb;
    const int tile = min(rb / 16, ntiles - 1);
    const WT* base = (MODE == kGateUp && rt == 1) ? w1 : w0;
    wp[rt] = base + static_cast<long long>(g) * a.w_group +
             static_cast<long long>(tile) * nkb * kFrag + lane * 8;
  }

  // token passes: workgroup z of nz takes passes z, z + nz, ... (a token's
  // arithmetic does not depend on which workgroup runs its pass)
  for (int m0 = bz * MT; m0 < M; m0 += nz * MT) {
    const int mp = min(MT, M - m0);
    // the branches are uniform across the workgroup
    if (mp <= 16) {
      gemm_pass_direct<WT, MODE, RT, MT, 1, W, KS>(a, lds, sel, off, m0, mp, wp, rowbase);
    } else if (mp <= 32) {
      gemm_pass_direct<WT, MODE, RT, MT, 2, W, KS>(a, lds, sel, off, m0, mp, wp, rowbase);
    } else if constexpr (NT >= 4) {
      if (mp <= 64 || NT == 4)
        gemm_pass_lds<WT, MODE, RT, MT, 4, W>(a, lds, sel, off, m0, mp, wp, rowbase);
      else
        gemm_pass_lds<WT, MODE, RT, MT, NT, W>(a, lds, sel, off, m0, mp, wp, rowbase);
    }
  }
}

template <typename WT, int MODE, int RT, int MT, int W, int KS = 1>
__global__ __launch_bounds__(W * 64) void stream_gemm(GemmArgs a) {
  stream_gemm_wg<WT, MODE, RT, MT, W, KS>(a, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.y, gridDim.z);
}

// ---------------------------------------------------------------------------
// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order:
// register arrays indexed by the constant stay in registers.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Tile schedule for large groups (prefill-sized batches).
//
// One workgroup computes one (group, column tile, BT-token tile).  Its 256
// weight rows (gate/up: 128 intermediate columns of gate and the same 128 of
// up; down: 256 hidden rows) and its BT token rows are staged in LDS one
// 32-wide K block at a time, both laid out as MFMA operand fragments (1 KB
// per 16 rows x 32 K for bf16): lane l of a fragment read takes the 16 bytes
// at l * 16, so operand reads are free of bank conflicts.  Weights are
// already fragment-packed in HBM; token rows are gathered into that layout by
// the load itself (lane (r, q) of a load fetches row r, elements 8q..8q+7 of
// the block).  Loads go straight from global memory to LDS
// (global_load_lds_dwordx4), kStages blocks deep, one barrier per block.
// Each wave multiplies 128 weight rows (8 fragments) against 64 tokens (4
// fragments): 32 MFMAs per block, 128 accumulator registers, so a SIMD holds
// two waves and one wave's MFMAs cover the other's waits.  BT = 256: 8 waves
// and one workgroup per CU; BT = 128: 4 waves, and two workgroups per CU
// whose epilogues (the output stores) overlap each other's MFMAs.
// Consecutive tiles land on the same XCD and, within a group, cover a block
// of token tiles x every column tile, so the workgroups sharing a weight slab
// or a token tile run side by side and read it through one L2.  Accumulation is the
// same single fp32 chain over K blocks in order with the same MFMA as the
// streaming schedule: results are bitwise identical.
constexpr int kMaxGroups = 64 + 8;       // routed + shared experts
constexpr int kTileBlock = 4;  // token tiles per ordering block
constexpr int kXcds = 8;

template <int MODE> constexpr int tile_cols() { return MODE == kGateUp ? 128 : 256; }  // output rows / 2 for gate/up

template <typename WT, int BT> struct TileCfg {
  static_assert(BT == 128 || BT == 256, "token tile");
  static constexpr int kWaves = 2 * BT / 64;                             // 2 x (BT / 64) grid
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kXFrags = BT / 16;                                // token fragments
  static constexpr int kFrags = 16 + kXFrags;                            // per K block
  static constexpr int kFragBytes = 512 * static_cast<int>(sizeof(WT));  // 16 x 32 operand block
  static constexpr int kDma = kFragBytes / 1024;                         // 16-B loads per lane
  // Token pairs (bf16, BT = 256).  A bf16 token row holds 64 B of one 32-wide
  // K block, half a 128-byte line.  With kXPair the token rows are staged two
  // K blocks at a time in a ring of two regions of their own, so that every
  // token load instruction reads 8 rows x 128 B, whole lines, while the
  // weight fragments keep their ring of kStages single-block stages (see
  // tile_gemm).
  static constexpr bool kXPair = sizeof(WT) == 2 && BT == 256;
  static constexpr int kStageBytes = (kXPair ? 16 : kFrags) * kFragBytes;
  static constexpr int kXRegionBytes = kXPair ? BT * 128 : 0;
  static constexpr int kWPerWave = 16 / kWaves;                          // fragments each wave loads
  static constexpr int kXPerWave = kXFrags / kWaves;
  // loads per lane: weight fragments per K block; token rows per K block,
  // or per pair of K blocks with kXPair
  static constexpr int kWLoads = kWPerWave * kDma;
  static constexpr int kXLoads = kXPair ? BT / 8 / kWaves : kXPerWave * kDma;
  // LDS: 160 KB per CU.  bf16 with BT = 128 keeps two workgroups per CU.
  static constexpr int kStages = sizeof(WT) == 4 ? 2 : (BT == 256 ? 4 : 3);
  static constexpr int kPerCu = (BT == 128 && sizeof(WT) == 2) ? 2 : 1;
  static_assert((kStages * kStageBytes + 2 * kXRegionBytes) * kPerCu <= 160 * 1024, "LDS budget");
  static_assert(!kXPair || (kDma == 1 && kStages == 4), "token pairs: bf16, four weight stages");
};

typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

// Workgroup barrier for the LDS pipeline: wait until at most N of this
// wave's vector-memory loads are outstanding (so its direct-to-LDS writes
// older than those have landed) and all its LDS reads are done, then
// s_barrier.  __syncthreads would also wait for the N newest loads, which
// are the prefetches the pipeline wants in flight across the barrier.  The
// empty asm statements keep the compiler from moving memory accesses across.
template <int N> __device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);  // lgkmcnt(0), expcnt off
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One LDS stage array per pipeline stage: separate objects let the compiler
// see that reading one stage does not wait for loads into another.
template <typename WT, int BT, int U> __device__ __forceinline__ unsigned char* tile_stage() {
  constexpr int B = TileCfg<WT, BT>::kStageBytes;
  __shared__ __attribute__((aligned(1024))) unsigned char s0[B];
  __shared__ __attribute__((aligned(1024))) unsigned char s1[B];
  __shared__ __attribute__((aligned(1024))) unsigned char s2[B];
  __shared__ __attribute__((aligned(1024))) unsigned char s3[B];
  static_assert(U >= 0 && U < 4, "at most four stages");
  if constexpr (U == 0) return s0;
  else if constexpr (U == 1) return s1;
  else if constexpr (U == 2) return s2;
  else return s3;
}

// The two token regions of the kXPair layout.
template <typename WT, int BT, int P> __device__ __forceinline__ unsigned char* tile_xregion() {
  constexpr int B = TileCfg<WT, BT>::kXRegionBytes > 0 ? TileCfg<WT, BT>::kXRegionBytes : 16;
  __shared__ __attribute__((aligned(1024))) unsigned char x0[B];
  __shared__ __attribute__((aligned(1024))) unsigned char x1[B];
  static_assert(P == 0 || P == 1, "two token regions");
  if constexpr (P == 0) return x0;
  else return x1;
}

// SETS: the groups are token sets (routed group g's rows from its mask,
// pairs from pinfo, act rows g*T + m) instead of moe_permute's order.
template <typename WT, int MODE, int BT, bool SETS = false>
__global__ __launch_bounds__((TileCfg<WT, BT>::kThreads), (TileCfg<WT, BT>::kPerCu)) void tile_gemm(
    GemmArgs a, int n_ctiles, int G) {
  using TC = TileCfg<WT, BT>;
  constexpr int kNS = TC::kStages;
  constexpr int kFB = TC::kFragBytes;
  constexpr int kNWT = BT / 64;          // waves along tokens
  __shared__ int group_start[kMaxGroups];  // first tile of each group
  __shared__ int group_tiles[kMaxGroups];  // tiles of each group
  __shared__ int group_mt[kMaxGroups];     // token tiles of each group
  __shared__ int tile_info[2][3];          // (group, column tile, token tile), two tiles in flight
  __shared__ int tile_total;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int ng = MODE == kHead ? 1 : G;

  // Tile counts per group (known on the device only): thread t counts group
  // t's tiles, then the start of its range from the counts before it.  The
  // LM head is one group of T tokens.
  if (tid < ng) {
    int M = a.T;
    if constexpr (SETS) {
      if (tid < a.E) M = set_size(a, tid);
    } else if (MODE != kHead) {
      M = max(0, min(a.offsets[tid + 1], a.P) - max(min(a.offsets[tid], a.P), 0));
    }
    const int mt = (M + BT - 1) / BT;
    group_mt[tid] = mt;
    group_tiles[tid] = mt * n_ctiles;
  }
  __syncthreads();
  if (tid < ng) {
    int run = 0;
    for (int u = 0; u < tid; ++u) run += group_tiles[u];
    group_start[tid] = run;
    if (tid == ng - 1) tile_total = run + group_tiles[tid];
  }
  __syncthreads();

  // The workgroups are persistent: hardware deals consecutive block ids
  // round-robin over the XCDs, so XCD x's workgroups walk the run of tiles
  // [x R, (x+1) R), R = ceil(tiles / 8), at a stride of their count: the
  // tiles an XCD works on at any moment are consecutive.  Within a group,
  // tiles run in blocks of kTileBlock token tiles x every column tile
  // (column-major inside the block): the ~32 tiles an XCD runs at once then
  // share both their weight slabs and their token rows in its L2.
  const int total = tile_total;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int stride = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int tile_end = min((xcd + 1) * per_xcd, total);
  int tile = xcd * per_xcd + blockIdx.x / kXcds;
  if (tile >= tile_end) return;

  // tile -> tile_info[buf] (every thread calls it; a barrier must follow)
  auto lookup = [&](int t, int buf) {
    if (tid < ng) {
      const int s0 = group_start[tid];
      if (t >= s0 && t < s0 + group_tiles[tid]) {
        const int r = t - s0;
        const int mtiles = group_mt[tid];
        const int mb0 = r / (kTileBlock * n_ctiles) * kTileBlock;
        const int rows = min(kTileBlock, mtiles - mb0);
        const int rr = r - mb0 * n_ctiles;
        const int ct = rr / rows;
        tile_info[buf][0] = tid;
        tile_info[buf][1] = ct;
        tile_info[buf][2] = mb0 + rr - ct * rows;
      }
    }
  };

  const int K = a.K;
  const int nkb = K / 32;
  const int last = nkb - 1;
  const int last_pair = nkb / 2 - 1;  // kXPair: K is a multiple of 64

  // the current tile: group, column tile, first token, token count, row base
  int g = 0, ct = 0, m0 = 0, mp = 0, off = 0;
  // This wave loads weight fragments wave*kWPerWave .. and token fragments
  // wave*kXPerWave .. of every block.  Token rows past the group's end
  // repeat its last row: MFMA output columns depend on their own token row
  // only, the epilogue drops those columns, and unconditional loads keep the
  // wait counts exact.
  //
  // Token pairs (kXPair): load instruction i (0..BT/8-1) of a pair covers
  // tokens 8i..8i+7 and the pair's 64 K values, 128 B per row.  Lane L
  // fetches row r = L / 8, 16-byte chunk c = (L % 8) ^ r ^ (i % 2), and the
  // load writes it to slot L of the instruction's 1 KB in LDS: slot
  // r*8 + (c ^ r ^ (i % 2)) holds (token 8i + r, chunk c).  A fragment read of
  // the pair's K block s (chunks 4s..4s+3) then has its 16 lanes of one chunk
  // on 16 distinct 16-byte bank groups.
  constexpr int kXPtr = TC::kXPair ? TC::kXLoads : TC::kXPerWave;
  const WT* wsrc[TC::kWPerWave];
  const WT* xsrc[kXPtr];
  auto setup = [&](int buf) {
    g = tile_info[buf][0];
    ct = tile_info[buf][1];
    int M;
    if constexpr (SETS) {
      off = g * a.T;
      M = g < a.E ? set_size(a, g) : a.T;
    } else {
      off = MODE == kHead ? 0 : clampi(a.offsets[g], 0, a.P);
      M = MODE == kHead ? a.T : clampi(a.offsets[g + 1], off, a.P) - off;
    }
    m0 = tile_info[buf][2] * BT;
    mp = min(BT, M - m0);
#pragma unroll
    for (int i = 0; i < TC::kWPerWave; ++i) {
      const int f = wave * TC::kWPerWave + i;  // 16-row weight tile f (0..15) of the tile
      int t;
      const WT* base;
      if (MODE == kGateUp) {  // f = 8 * half + 4 * (up ? 1 : 0) + i
        t = ct * (tile_cols<MODE>() / 16) + (f >> 3) * 4 + (f & 3);
        base = static_cast<const WT*>((f & 4) ? a.w1 : a.w0);
      } else if (MODE == kHead) {  // the last column tile may run past the vocabulary
        t = min(ct * (tile_cols<MODE>() / 16) + f, (a.N + 15) / 16 - 1);
        base = static_cast<const WT*>(a.w0);
      } else {
        t = ct * (tile_cols<MODE>() / 16) + f;
        base = static_cast<const WT*>(a.w0);
      }
      wsrc[i] = base + static_cast<long long>(g) * a.w_group + static_cast<long long>(t) * nkb * 512 + lane * 8;
    }
    if constexpr (TC::kXPair) {
#pragma unroll
      for (int i = 0; i < kXPtr; ++i) {
        const int ii = wave * kXPtr + i;  // load instruction of the pair
        const int r = lane >> 3;
        const int row = min(ii * 8 + r, mp - 1);
        const int c = (lane & 7) ^ r ^ (ii & 1);
        xsrc[i] = static_cast<const WT*>(a.x) + tile_row<MODE, SETS>(a, g, off, m0, row) * K + c * 8;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kXPtr; ++i) {
        const int row = min((wave * TC::kXPerWave + i) * 16 + r16, mp - 1);
        xsrc[i] = static_cast<const WT*>(a.x) + tile_row<MODE, SETS>(a, g, off, m0, row) * K + q * 8;
      }
    }
  };
  // token pair pr (K blocks 2pr, 2pr+1) into region P (kXPair)
  auto issue_x = [&](auto P, int pr) __attribute__((always_inline)) {
    unsigned char* xr = tile_xregion<WT, BT, decltype(P)::value>();
#pragma unroll
    for (int i = 0; i < kXPtr; ++i)
      __builtin_amdgcn_global_load_lds((gptr_t)(xsrc[i] + pr * 64), (lptr_t)(xr + (wave * kXPtr + i) * 1024), 16,
                                       0, 0);
  };
  // K block kb into stage U: for each fragment, kDma loads of 16 B per lane
  // (the weights only with kXPair)
  auto issue = [&](auto U, int kb) __attribute__((always_inline)) {
    unsigned char* st = tile_stage<WT, BT, decltype(U)::value>();
    if constexpr (TC::kXPair) {
#pragma unroll
      for (int i = 0; i < TC::kWPerWave; ++i)
        __builtin_amdgcn_global_load_lds((gptr_t)(wsrc[i] + kb * 512),
                                         (lptr_t)(st + (wave * TC::kWPerWave + i) * kFB), 16, 0, 0);
      return;
    }
#pragma unroll
    for (int h = 0; h < TC::kDma; ++h) {
#pragma unroll
      for (int i = 0; i < TC::kWPerWave; ++i)
        __builtin_amdgcn_global_load_lds((gptr_t)(wsrc[i] + kb * 512 + h * (16 / sizeof(WT))),
                                         (lptr_t)(st + (wave * TC::kWPerWave + i) * kFB + h * 1024), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < TC::kXPerWave; ++i)
        __builtin_amdgcn_global_load_lds((gptr_t)(xsrc[i] + kb * 32 + h * (16 / sizeof(WT))),
                                         (lptr_t)(st + (16 + wave * TC::kXPerWave + i) * kFB + h * 1024), 16,
                                         0, 0);
    }
  };
  // loads per lane per block (without kXPair)
  constexpr int kLoads = TC::kWLoads + TC::kXLoads;
  // blocks 0 .. kNS-2 of the tile set up last (clamped: K may hold fewer);
  // with kXPair the first token pair goes first
  auto prologue = [&]() __attribute__((always_inline)) {
    if constexpr (TC::kXPair) issue_x(std::integral_constant<int, 0>{}, 0);
    static_for<kNS - 1>([&](auto U) __attribute__((always_inline)) { issue(U, min(decltype(U)::value, last)); });
  };
  // Wait counts (loads complete in order).  Without kXPair: block kb + 1 has
  // landed once at most the kNS - 2 newer blocks' loads are outstanding.  With
  // kXPair, iteration kb requests weight block kb + 3 and, for even kb, token
  // pair kb/2 + 1; at its end block kb + 1 needs weight block kb + 1 (three
  // iterations old) and token pair (kb + 1)/2 (requested at iteration
  // kb - 2 for odd kb + 1, at kb - 1 for even kb + 1): even kb may leave its
  // own and iteration kb - 1's requests outstanding, odd kb only its own.
  constexpr int kWaitTop = TC::kXPair ? (kNS - 2) * TC::kWLoads : (kNS - 2) * kLoads;
  constexpr int kWaitEven = TC::kXPair ? 2 * TC::kWLoads + TC::kXLoads : (kNS - 2) * kLoads;
  constexpr int kWaitOdd = TC::kXPair ? TC::kWLoads : (kNS - 2) * kLoads;

  const int wr = wave / kNWT;  // weight half
  const int wt = wave % kNWT;  // token quarter (BT = 256) or half (BT = 128)
  // fragment reads: lane l takes 16 B at l * 16 of each kDma half
  auto frag = [&](const unsigned char* st, int f, Frag<WT>& out) __attribute__((always_inline)) {
    if constexpr (sizeof(WT) == 2) {
      out.v = *reinterpret_cast<const bf16x8*>(st + f * kFB + lane * 16);
    } else {
      out.lo = *reinterpret_cast<const f32x4*>(st + f * kFB + lane * 16);
      out.hi = *reinterpret_cast<const f32x4*>(st + f * kFB + 1024 + lane * 16);
    }
  };

  // kXPair: this lane's byte offsets, in a token region, of its fragments of
  // the pair's K block s (token column wt*64 + j*16 + r16 sits at + j * 2048)
  int xoff[2];
  if constexpr (TC::kXPair) {
    const int h = (lane >> 3) & 1, r = lane & 7;
#pragma unroll
    for (int s = 0; s < 2; ++s) xoff[s] = (wt * 8 + h) * 1024 + (r * 8 + ((s * 4 + q) ^ r ^ h)) * 16;
  }

  f32x4 acc[8][4];
  // Block kb sits in stage kb % kNS (its token rows, with kXPair, in region
  // (kb / 2) % 2).  Iteration kb requests block kb + kNS - 1 into the stage
  // read in the previous iteration (and, for even kb with kXPair, token pair
  // kb/2 + 1 into the region the previous pair used), multiplies block kb,
  // then waits until block kb + 1 has landed (its loads and those of every
  // other wave: the barrier).  Iterations run in groups of kNS from a
  // multiple of kNS, so kb % kNS = U and, with kXPair, kb % 2 = U % 2 and
  // (kb / 2) % 2 = U / 2.
  auto iteration = [&](auto U, int kb) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    issue(std::integral_constant<int, (u + kNS - 1) % kNS>{}, min(kb + kNS - 1, last));
    if constexpr (TC::kXPair && u % 2 == 0)
      issue_x(std::integral_constant<int, (u / 2 + 1) % 2>{}, min(kb / 2 + 1, last_pair));
    // Keep the requests at the top of the iteration: the scheduler would
    // otherwise sink them to the wait at its end.
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char* st = tile_stage<WT, BT, u>();
    Frag<WT> A[8], B[4];
    if constexpr (TC::kXPair) {
      const unsigned char* xr = tile_xregion<WT, BT, (u / 2) % 2>();
#pragma unroll
      for (int j = 0; j < 4; ++j) B[j].v = *reinterpret_cast<const bf16x8*>(xr + xoff[u % 2] + j * 2048);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) frag(st, 16 + wt * 4 + j, B[j]);
    }
    // While direct-to-LDS loads are in flight (always, in this loop) the
    // compiler waits for every outstanding LDS read before an MFMA that needs
    // one, so the weight fragments are read in batches ahead of their MFMAs:
    // kAhead row tiles ahead (two for 256-token tiles, all eight up front for
    // 128-token tiles; the fastest of 2, 3, 4 and 8 measured for each).  The
    // group barriers keep that order.
    constexpr int kAhead = BT == 256 ? 2 : 8;
    constexpr int kRd = sizeof(WT) == 2 ? 1 : 2;  // LDS reads per fragment
#pragma unroll
    for (int rt = 0; rt < kAhead; ++rt) frag(st, wr * 8 + rt, A[rt]);
    __builtin_amdgcn_sched_group_barrier(0x100, (4 + kAhead) * kRd, 0);  // DS reads
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      if (rt + kAhead < 8) {
        frag(st, wr * 8 + rt + kAhead, A[rt + kAhead]);
        __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[rt][j] = mma(A[rt], B[j], acc[rt][j]);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMAs
    }
    stage_barrier<(u % 2 == 0) ? kWaitEven : kWaitOdd>();
  };

  lookup(tile, 0);
  __syncthreads();
  int cur = 0;
  setup(cur);
  prologue();
  for (;;) {
    // Stage 0 of this tile has landed.  After an epilogue its stores are
    // newer than the prologue's loads, so this waits for them too: correct,
    // a little early.
    stage_barrier<kWaitTop>();
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    int kb0 = 0;
    for (; kb0 + kNS <= nkb; kb0 += kNS)
      static_for<kNS>([&](auto U) __attribute__((always_inline)) { iteration(U, kb0 + decltype(U)::value); });
    static_for<kNS>([&](auto U) __attribute__((always_inline)) {
      if (kb0 + decltype(U)::value < nkb) iteration(U, kb0 + decltype(U)::value);
    });
    stage_barrier<0>();  // clamped tail loads; every stage is free again

    // The next tile's first blocks are requested before this tile's
    // epilogue, so their latency overlaps the epilogue's math and stores.
    const int e_g = g, e_ct = ct, e_m0 = m0, e_mp = mp, e_off = off;
    const int next = tile + stride;
    const bool more = next < tile_end;
    if (more) {
      lookup(next, cur ^ 1);
      __syncthreads();
      cur ^= 1;
      setup(cur);
      prologue();
    }

    // epilogue: lane (r16, q) holds weight rows 4q + v of fragment wr*8 + rt
    // for token column wt*64 + j*16 + r16
    if constexpr (MODE == kGateUp) {
      WT* act = static_cast<WT*>(a.out);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = wt * 64 + j * 16 + r16;
        if (m < e_mp) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 gv = acc[i][j], uv = acc[4 + i][j];
            f32x4 o;
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = silu_mul(gv[v], uv[v]);
            const int col = e_ct * tile_cols<MODE>() + wr * 64 + i * 16 + 4 * q;
            store4<WT>(act + static_cast<long long>(e_off + e_m0 + m) * a.N + col, o);
          }
        }
      }
    } else if constexpr (MODE == kHead) {
      // per token column: best (value, vocab index) over this wave's 128
      // rows, then over the two waves sharing the column (LDS), written as
      // partial block e_ct of the arg max
      __shared__ float red_v[2 * BT];
      __shared__ int red_i[2 * BT];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = wt * 64 + j * 16 + r16;
        float best = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = e_ct * tile_cols<MODE>() + (wr * 8 + rt) * 16 + 4 * q + v;
            if (n < a.N) {
              const float val = acc[rt][j][v];
              if (a.logits != nullptr && m < e_mp) a.logits[static_cast<long long>(e_m0 + m) * a.N + n] = val;
              if (better(val, n, best, bi)) { best = val; bi = n; }
            }
          }
#pragma unroll
        for (int msk = 16; msk <= 32; msk <<= 1) {
          const float ov = __shfl_xor(best, msk, kWave);
          const int oi = __shfl_xor(bi, msk, kWave);
          if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
        }
        if (q == 0) {
          red_v[wr * BT + m] = best;
          red_i[wr * BT + m] = bi;
        }
      }
      stage_barrier<63>();  // LDS writes visible; the prologue's loads stay in flight
      if (tid < e_mp) {
        float best = red_v[tid];
        int bi = red_i[tid];
        if (better(red_v[BT + tid], red_i[BT + tid], best, bi)) {
          best = red_v[BT + tid];
          bi = red_i[BT + tid];
        }
        const long long o = static_cast<long long>(e_m0 + tid) * n_ctiles + e_ct;  // [T][blocks]
        static_cast<float*>(a.out)[o] = best;
        a.out_idx[o] = bi;
      }
      stage_barrier<63>();  // red_* free for the next tile
    } else {
      float* y = static_cast<float*>(a.out);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = wt * 64 + j * 16 + r16;
        if (m < e_mp) {
          int p;
          float wgt;
          if constexpr (SETS) {
            int t, slot;
            wgt = 1.0f;
            if (e_g < a.E) {
              t = set_nth(a, e_g, e_m0 + m);
              const int2 pi = a.pinfo[static_cast<long long>(t) * a.E + e_g];
              slot = clampi(pi.y, 0, a.k - 1);
              wgt = __int_as_float(pi.x);
            } else {
              t = e_m0 + m;
              slot = a.k + e_g - a.E;
            }
            p = t * a.S + slot;
          } else {
            p = clampi(a.sorted_src[e_off + e_m0 + m], 0, a.P - 1);
            const int t = p / a.S;
            const int slot = p - t * a.S;
            wgt = slot < a.k ? a.topk_w[static_cast<long long>(t) * a.k + slot] : 1.0f;
          }
#pragma unroll
          for (int rt = 0; rt < 8; ++rt) {
            f32x4 o = acc[rt][j];
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] *= wgt;
            const int row = e_ct * tile_cols<MODE>() + (wr * 8 + rt) * 16 + 4 * q;
            store4<float>(y + static_cast<long long>(p) * a.N + row, o);
          }
        }
      }
    }
    (void)e_g;
    if (!more) break;
    tile = next;
  }
}

// Persistent workgroups: one per CU slot (two per CU for 128-token tiles),
// at most one per tile of the upper bound (groups are only known on the
// device: every group contributes at most ceil(M_g / BT) <= M_g / BT + 1
// token tiles); a multiple of the XCD count.
int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

int tile_grid(int T, int k, int ns, int E, int n_ctiles, int BT, int per_cu) {
  const long long routed = (static_cast<long long>(T) * k + BT - 1) / BT + E;
  const long long shared = static_cast<long long>(ns) * ((T + BT - 1) / BT);
  long long n = std::min<long long>((routed + shared) * n_ctiles, static_cast<long long>(cu_count()) * per_cu);
  n = (n + kXcds - 1) / kXcds * kXcds;
  return static_cast<int>(n);
}

// 256-token tiles once routed groups average 384 tokens or more (less
// padding in ragged last tiles below that).
template <typename WT, int MODE, bool SETS = false>
void launch_tile(const GemmArgs& args, int n_ctiles, int G, int E, int k, int ns, hipStream_t s) {
  // token sets reach at most kSetMaxTokens rows: always 128-token tiles
  if (!SETS && static_cast<long long>(args.T) * k >= 384LL * E && (!TileCfg<WT, 256>::kXPair || args.K % 64 == 0)) {
    const int grid = tile_grid(args.T, k, ns, E, n_ctiles, 256, TileCfg<WT, 256>::kPerCu);
    tile_gemm<WT, MODE, 256><<<grid, TileCfg<WT, 256>::kThreads, 0, s>>>(args, n_ctiles, G);
  } else {
    const int grid = tile_grid(args.T, k, ns, E, n_ctiles, 128, TileCfg<WT, 128>::kPerCu);
    tile_gemm<WT, MODE, 128, SETS><<<grid, TileCfg<WT, 128>::kThreads, 0, s>>>(args, n_ctiles, G);
  }
}

// LM head on the tile schedule: one group of T tokens, 256 vocabulary rows
// per column tile, so the partial arg max blocks are the column tiles.
constexpr int kHeadTileMinTokens = 32;
static_assert(tile_cols<kHead>() == 16 * kRtHead * kWavesHead, "head partial blocks");

template <typename WT>
void launch_tile_head(const GemmArgs& args, int n_ctiles, hipStream_t s) {
  // 256-token tiles (one workgroup per CU) above 128 tokens: each column tile's
  // weights are then read once up to 256 tokens
  const int BT = (args.T > 128 && (!TileCfg<WT, 256>::kXPair || args.K % 64 == 0)) ? 256 : 128;
  long long n = std::min<long long>(static_cast<long long>(n_ctiles) * ((args.T + BT - 1) / BT),
                                    static_cast<long long>(cu_count()) * (BT == 256 ? TileCfg<WT, 256>::kPerCu
                                                                                    : TileCfg<WT, 128>::kPerCu));
  n = (n + kXcds - 1) / kXcds * kXcds;
  if (BT == 256)
    tile_gemm<WT, kHead, 256><<<static_cast<int>(n), TileCfg<WT, 256>::kThreads, 0, s>>>(args, n_ctiles, 1);
  else
    tile_gemm<WT, kHead, 128><<<static_cast<int>(n), TileCfg<WT, 128>::kThreads, 0, s>>>(args, n_ctiles, 1);
}

// Fragment packing of row-major weights: thread i writes the 8 elements of
// packed position i = ((g * ntiles + tile) * nkb + kb) * 64 + lane, taken from
// row tile*16 + lane % 16, columns kb*32 + 8*(lane / 16) .. +7 (zero past N).
template <typename WT>
__global__ __launch_bounds__(256) void pack_kernel(const WT* __restrict__ src, WT* __restrict__ dst,
                                                   int G, int N, int K) {
  const long long ntiles = (N + 15) / 16, nkb = K / 32;
  const long long total = static_cast<long long>(G) * ntiles * nkb * 64;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int lane = static_cast<int>(i & 63);
    long long r = i >> 6;
    const long long kb = r % nkb;
    r /= nkb;
    const long long tile = r % ntiles;
    const long long g = r / ntiles;
    const long long row = tile * 16 + (lane & 15);
    const long long col = kb * 32 + 8 * (lane >> 4);
    uint4* d = reinterpret_cast<uint4*>(dst + i * 8);
    constexpr int kVec = 8 * sizeof(WT) / 16;   // 16-byte vectors per 8 elements
    if (row < N) {
      const uint4* s = reinterpret_cast<const uint4*>(src + (g * N + row) * K + col);
#pragma unroll
      for (int v = 0; v < kVec; ++v) d[v] = s[v];
    } else {
#pragma unroll
      for (int v = 0; v < kVec; ++v) d[v] = make_uint4(0, 0, 0, 0);
    }
  }
}

// Final RMSNorm of the head input, rounded to the operand type.  With y (the
// last layer's expert slots) the residual add happens first, in the same slot
// order as the combine kernel.  TPB = 1 (decode sizes): 512 threads per
// token, every load issued before any is used and none under a per-slot
// branch (two staging passes cover H <= 4096; slot loads unrolled to SL >=
// S, entries past S repeat slot S - 1 and are not summed), and the RMSNorm
// gain requested first, kept raw until the scale is known.  TPB = 4: 256
// threads stage four rows pass by pass.
constexpr int kNormMaxSlots = 16;
constexpr int kNormMaxChunks = 12;  // 256-wide chunks of a row, H <= 3072

template <int TPB> constexpr int norm_threads() { return TPB == 1 ? 512 : 256; }

template <typename WT, int TPB, int SL>
__global__ __launch_bounds__(512) void norm_cast_kernel(const float* __restrict__ h,
                                                        const float* __restrict__ y, int S,
                                                        const WT* __restrict__ gamma, float eps,
                                                        int T, int H, WT* __restrict__ xo,
                                                        float* __restrict__ h_out) {
  extern __shared__ float hs[];   // [TPB][H]
  constexpr int kThreads = norm_threads<TPB>();
  const int t0 = blockIdx.x * TPB;
  const int nt = min(TPB, T - t0);
  const int h4 = H / 4;
  const int nch = (H + 255) / 256;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const bool norm_wave = wave < nt;
  // gain of this wave's row: lane covers elements c*256 + lane*4 .. +3
  typename GainRaw<WT>::T graw[kNormMaxChunks];
  if (norm_wave && gamma != nullptr) {
#pragma unroll
    for (int c = 0; c < kNormMaxChunks; ++c)
      if (c < nch) graw[c] = GainRaw<WT>::load(gamma + min(c * 256 + lane * 4, H - 4));
  }
  // residual (h, optional) plus the slots of row t at column i; returns it
  auto stage = [&](float4 v, const float4 (&sv)[SL], long long t, int tt, int i, bool store_h) {
    if (y != nullptr) {
      float4 acc = sv[0];
#pragma unroll
      for (int sl = 1; sl < SL; ++sl)
        if (sl < S) {
          acc.x += sv[sl].x;
          acc.y += sv[sl].y;
          acc.z += sv[sl].z;
          acc.w += sv[sl].w;
        }
      v = h != nullptr ? make_float4(v.x + acc.x, v.y + acc.y, v.z + acc.z, v.w + acc.w) : acc;
    }
    if (store_h && h_out != nullptr) *reinterpret_cast<float4*>(h_out + t * H + i) = v;
    *reinterpret_cast<float4*>(hs + tt * H + i) = v;
    return v;
  };
  auto load = [&](float4& v, float4 (&sv)[SL], long long t, int i) {
    v = h != nullptr ? *reinterpret_cast<const float4*>(h + t * H + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    if (y != nullptr) {
      const float4* ys = reinterpret_cast<const float4*>(y + t * S * H + i);
#pragma unroll
      for (int sl = 0; sl < SL; ++sl) sv[sl] = ys[static_cast<long long>(min(sl, S - 1)) * h4];
    }
  };
  // TPB = 1: the new residual is stored after the barrier (and, by the norm
  // wave, after its output), so no wait for a load is also a wait for it
  const int f0 = threadIdx.x, f1 = threadIdx.x + kThreads;
  float4 hk0, hk1;
  auto store_residual = [&]() {
    if constexpr (TPB == 1) {
      if (h_out != nullptr) {
        if (f0 < h4) *reinterpret_cast<float4*>(h_out + static_cast<long long>(t0) * H + f0 * 4) = hk0;
        if (f1 < h4) *reinterpret_cast<float4*>(h_out + static_cast<long long>(t0) * H + f1 * 4) = hk1;
      }
    }
  };
  if constexpr (TPB == 1) {
    float4 v0, v1, s0[SL], s1[SL];
    if (f0 < h4) load(v0, s0, t0, f0 * 4);
    if (f1 < h4) load(v1, s1, t0, f1 * 4);
    if (f0 < h4) hk0 = stage(v0, s0, t0, 0, f0 * 4, false);
    if (f1 < h4) hk1 = stage(v1, s1, t0, 0, f1 * 4, false);
  } else {
    for (int f = threadIdx.x; f < nt * h4; f += kThreads) {
      const int tt = f / h4;
      const int i = (f - tt * h4) * 4;
      float4 v, sv[SL];
      load(v, sv, t0 + tt, i);
      stage(v, sv, t0 + tt, tt, i, true);
    }
  }
  __syncthreads();
  if (!norm_wave) {
    store_residual();
    return;
  }
  const float* hr = hs + wave * H;
  float ss = 0.f;
  for (int i = lane * 4; i < H; i += 256) {
    const float4 v = *reinterpret_cast<const float4*>(hr + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = lane63(wave_sum_lane63(ss));
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
#pragma unroll
  for (int c = 0; c < kNormMaxChunks; ++c) {
    const int i = c * 256 + lane * 4;
    if (c < nch && i < H) {
      const float4 v = *reinterpret_cast<const float4*>(hr + i);
      const float4 g = gamma != nullptr ? GainRaw<WT>::to_f4(graw[c]) : make_float4(1.f, 1.f, 1.f, 1.f);
      f32x4 o;
      o[0] = v.x * r * g.x;
      o[1] = v.y * r * g.y;
      o[2] = v.z * r * g.z;
      o[3] = v.w * r * g.w;
      store4<WT>(xo + static_cast<long long>(t0 + wave) * H + i, o);
    }
  }
  store_residual();
}

// Second pass of the blocked arg max: one wavefront per token.
__global__ __launch_bounds__(64) void argmax_reduce_kernel(const float* __restrict__ pmax,
                                                           const int32_t* __restrict__ pidx,
                                                           int nblk, int T,
                                                           int32_t* __restrict__ argmax_out,
                                                           int out_stride,
                                                           float* __restrict__ max_out) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int b = lane; b < nblk; b += 64) {
    const float v = pmax[static_cast<long long>(t) * nblk + b];
    const int i = pidx[static_cast<long long>(t) * nblk + b];
    if (better(v, i, best, bi)) { best = v; bi = i; }
  }
  wave_argmax(best, bi);
  if (lane == 0) {
    argmax_out[static_cast<long long>(t) * out_stride] = bi;
    if (max_out) max_out[t] = best;
  }
}

// One block per sequence: wave j reduces row b*(K+1) + j exactly as
// argmax_reduce_kernel does, then one thread applies the prefix acceptance to
// the sequence's K+1 greedy tokens (K + 1 <= 16).
constexpr int kVerifyFuseMaxRows = 16;
__global__ __launch_bounds__(64 * kVerifyFuseMaxRows) void argmax_verify_kernel(const float* __restrict__ pmax,
                                                                              const int32_t* __restrict__ pidx,
                                                                              int nblk,
                                                                              int32_t* __restrict__ greedy,
                                                                              VerifyFuse v) {
  __shared__ int32_t tok_s[kVerifyFuseMaxRows];
  __shared__ int32_t gr_s[kVerifyFuseMaxRows];
  const int b = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int K1 = v.K + 1;
  const long long t = static_cast<long long>(b) * K1 + wave;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int blk = lane; blk < nblk; blk += 64) {
    const float val = pmax[t * nblk + blk];
    const int i = pidx[t * nblk + blk];
    if (better(val, i, best, bi)) { best = val; bi = i; }
  }
  wave_argmax(best, bi);
  if (lane == 0) {
    greedy[t] = bi;
    gr_s[wave] = bi;
    tok_s[wave] = v.tokens[t];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (v.pos != nullptr && (v.pos[b] < 0 || v.pos[b] > v.max_len - K1)) {
      // no room in the sequence's cache: nothing accepted or committed
      for (int j = 0; j < K1; ++j) v.commit[static_cast<long long>(b) * K1 + j] = -1;
      v.n_accept[b] = -1;
      if (v.commit_len) v.commit_len[b] = 0;
      if (v.next_last) v.next_last[b] = tok_s[0];
      return;
    }
    const int n = accept_prefix(tok_s, gr_s, v.K, v.commit + static_cast<long long>(b) * K1);
    v.n_accept[b] = n;
    if (v.commit_len) v.commit_len[b] = n + 1;
    if (v.next_last) v.next_last[b] = gr_s[n];
  }
}

// Token-pass variant by batch size: every group holds at most T rows (the
// shared experts hold exactly T), so T <= MT means one pass per group.
template <typename WT, int MODE, int RT, int W>
void launch_gemm(const GemmArgs& args, dim3 grid, hipStream_t s) {
  if (args.T <= 32)
    stream_gemm<WT, MODE, RT, 32, W><<<grid, W * 64, 0, s>>>(args);
  else if (args.T <= 64)
    stream_gemm<WT, MODE, RT, 64, W><<<grid, W * 64, 0, s>>>(args);
  else
    stream_gemm<WT, MODE, RT, 128, W><<<grid, W * 64, 0, s>>>(args);
}

int head_blocks(int V) { return (V + 16 * kRtHead * kWavesHead - 1) / (16 * kRtHead * kWavesHead); }

size_t esize(int dt) { return dt == MOEV_BF16 ? 2 : 4; }

moev_status check_inter(int I) {
  MOEV_REQUIRE(I >= 64 && I <= 8192 && I % 64 == 0, MOEV_ERR_UNSUPPORTED,
               "intermediate size %d must be a multiple of 64 in [64, 8192]", I);
  return MOEV_OK;
}

moev_status check_hid(int H) {
  MOEV_REQUIRE(H >= 64 && H <= 3072 && H % 64 == 0, MOEV_ERR_UNSUPPORTED,
               "hidden size %d must be a multiple of 64 in [64, 3072]", H);
  return MOEV_OK;
}

}  // namespace

size_t grouped_ffn_ws_bytes(int T, int I, int k, int ns, int dt) {
  return align_up(static_cast<size_t>(T) * (k + ns) * I * esize(dt), 256);
}

size_t lmhead_ws_bytes(int T, int H, int V, int dt) {
  const size_t xf = align_up(static_cast<size_t>(T) * H * esize(dt), 256);
  const size_t part = align_up(static_cast<size_t>(head_blocks(V)) * T * 4, 256);
  return xf + 2 * part;
}

GemmArgs ffn_args(const int32_t* sorted_src, const int32_t* offsets, int T, int H, int I,
                  int k, int ns) {
  GemmArgs a{};
  a.offsets = offsets;
  a.sorted_src = sorted_src;
  a.S = k + ns;
  a.k = k;
  a.P = T * (k + ns);
  a.T = T;
  a.n_first = ns;
  return a;
}

void launch_ffn_gate_up(const void* x, const int32_t* sorted_src, const int32_t* offsets,
                        const void* w_gate, const void* w_up, int T, int H, int I, int E, int k,
                        int ns, int dt, void* act, hipStream_t s) {
  GemmArgs up = ffn_args(sorted_src, offsets, T, H, I, k, ns);
  up.w0 = w_gate;
  up.w1 = w_up;
  up.w_group = static_cast<long long>(I) * H;
  up.N = I;
  up.K = H;
  up.x = x;
  up.out = act;
  if (T > kTileMinTokens && I % tile_cols<kGateUp>() == 0) {
    const int nct = I / tile_cols<kGateUp>();
    if (dt == MOEV_BF16) launch_tile<u16, kGateUp>(up, nct, E + ns, E, k, ns, s);
    else launch_tile<float, kGateUp>(up, nct, E + ns, E, k, ns, s);
    return;
  }
  const dim3 grid(I / (16 * kWavesFfn), E + ns);
  if (dt == MOEV_BF16)
    launch_gemm<u16, kGateUp, 2, kWavesFfn>(up, grid, s);
  else
    launch_gemm<float, kGateUp, 2, kWavesFfn>(up, grid, s);
}

void launch_ffn_down(const void* act, const int32_t* sorted_src, const int32_t* offsets,
                     const float* topk_w, const void* w_down, int T, int H, int I, int E, int k,
                     int ns, int dt, float* y_slots, hipStream_t s) {
  GemmArgs dn = ffn_args(sorted_src, offsets, T, H, I, k, ns);
  dn.w0 = w_down;
  dn.w_group = static_cast<long long>(H) * I;
  dn.N = H;
  dn.K = I;
  dn.x = act;
  dn.topk_w = topk_w;
  dn.out = y_slots;
  if (T > kTileMinTokens && H % tile_cols<kDown>() == 0) {
    const int nct = H / tile_cols<kDown>();
    if (dt == MOEV_BF16) launch_tile<u16, kDown>(dn, nct, E + ns, E, k, ns, s);
    else launch_tile<float, kDown>(dn, nct, E + ns, E, k, ns, s);
    return;
  }
  const dim3 grid(H / (16 * kRtDown * kWavesFfn), E + ns);
  if (dt == MOEV_BF16)
    launch_gemm<u16, kDown, kRtDown, kWavesFfn>(dn, grid, s);
  else
    launch_gemm<float, kDown, kRtDown, kWavesFfn>(dn, grid, s);
}

GemmArgs set_args(const uint64_t* masks, const int2* pinfo, int T, int H, int I, int E, int k, int ns) {
  GemmArgs a = ffn_args(nullptr, nullptr, T, H, I, k, ns);
  a.sets = true;
  a.E = E;
  a.W = (T + 63) / 64;
  a.masks = masks;
  a.pinfo = pinfo;
  return a;
}

void launch_ffn_gate_up_sets(const void* x, const uint64_t* masks, const void* w_gate,
                             const void* w_up, int T, int H, int I, int E, int k, int ns, int dt,
                             void* act, hipStream_t s, bool split_k) {
  GemmArgs up = set_args(masks, nullptr, T, H, I, E, k, ns);
  up.w0 = w_gate;
  up.w1 = w_up;
  up.w_group = static_cast<long long>(I) * H;
  up.N = I;
  up.K = H;
  up.x = x;
  up.out = act;
  if (split_k) {
    const dim3 grid(I / 16, E + ns);
    if (dt == MOEV_BF16)
      stream_gemm<u16, kGateUp, 2, 32, kWavesFfn, kWavesFfn><<<grid, kWavesFfn * 64, 0, s>>>(up);
    else
      stream_gemm<float, kGateUp, 2, 32, kWavesFfn, kWavesFfn><<<grid, kWavesFfn * 64, 0, s>>>(up);
    return;
  }
  if (T > kTileMinTokens) {  // sets_fit: I is a whole number of column tiles
    const int nct = I / tile_cols<kGateUp>();
    if (dt == MOEV_BF16) launch_tile<u16, kGateUp, true>(up, nct, E + ns, E, k, ns, s);
    else launch_tile<float, kGateUp, true>(up, nct, E + ns, E, k, ns, s);
    return;
  }
  const dim3 grid(I / (16 * kWavesFfn), E + ns);
  if (dt == MOEV_BF16)
    launch_gemm<u16, kGateUp, 2, kWavesFfn>(up, grid, s);
  else
    launch_gemm<float, kGateUp, 2, kWavesFfn>(up, grid, s);
}

void launch_ffn_down_sets(const void* act, const uint64_t* masks, const int2* pinfo,
                          const void* w_down, int T, int H, int I, int E, int k, int ns, int dt,
                          float* y_slots, hipStream_t s, bool split_k, int pass_split,
                          const QkvScatter* scatter) {
  GemmArgs dn = set_args(masks, pinfo, T, H, I, E, k, ns);
  dn.w0 = w_down;
  dn.w_group = static_cast<long long>(H) * I;
  dn.N = H;
  dn.K = I;
  dn.x = act;
  dn.out = y_slots;
  if (scatter != nullptr) {
    dn.scatter = *scatter;
    dn.scattered = true;
  }
  // dense projections of a whole batch (pass_split > 1): two 16-row tiles per
  // workgroup halve the operand rows' L2 re-reads; the K order of every output
  // is unchanged
  if (split_k && pass_split > 1 && H % 32 == 0) {
    const int z = max(1, min(pass_split, (T + 31) / 32));
    const dim3 grid(H / 32, E + ns, z);
    if (dt == MOEV_BF16)
      stream_gemm<u16, kDown, 2, 32, kWavesFfn, kWavesFfn><<<grid, kWavesFfn * 64, 0, s>>>(dn);
    else
      stream_gemm<float, kDown, 2, 32, kWavesFfn, kWavesFfn><<<grid, kWavesFfn * 64, 0, s>>>(dn);
    return;
  }
  if (split_k) {
    const int z = max(1, min(pass_split, (T + 31) / 32));
    const dim3 grid(H / (16 * kRtDown), E + ns, z);
    if (dt == MOEV_BF16)
      stream_gemm<u16, kDown, kRtDown, 32, kWavesFfn, kWavesFfn><<<grid, kWavesFfn * 64, 0, s>>>(dn);
    else
      stream_gemm<float, kDown, kRtDown, 32, kWavesFfn, kWavesFfn><<<grid, kWavesFfn * 64, 0, s>>>(dn);
    return;
  }
  if (T > kTileMinTokens) {  // sets_fit: H is a whole number of column tiles
    const int nct = H / tile_cols<kDown>();
    if (dt == MOEV_BF16) launch_tile<u16, kDown, true>(dn, nct, E + ns, E, k, ns, s);
    else launch_tile<float, kDown, true>(dn, nct, E + ns, E, k, ns, s);
    return;
  }
  const dim3 grid(H / (16 * kRtDown * kWavesFfn), E + ns);
  if (dt == MOEV_BF16)
    launch_gemm<u16, kDown, kRtDown, kWavesFfn>(dn, grid, s);
  else
    launch_gemm<float, kDown, kRtDown, kWavesFfn>(dn, grid, s);
}

bool sets_fit(int T, int H, int I) {
  return T <= kTileMinTokens ||
         (T <= kSetMaxTokens && I % tile_cols<kGateUp>() == 0 && H % tile_cols<kDown>() == 0);
}

void launch_grouped_ffn(const void* x, const int32_t* sorted_src, const int32_t* offsets,
                        const float* topk_w, const void* w_gate, const void* w_up,
                        const void* w_down, int T, int H, int I, int E, int k, int ns, int dt,
                        float* y_slots, void* ws, hipStream_t s) {
  launch_ffn_gate_up(x, sorted_src, offsets, w_gate, w_up, T, H, I, E, k, ns, dt, ws, s);
  launch_ffn_down(ws, sorted_src, offsets, topk_w, w_down, T, H, I, E, k, ns, dt, y_slots, s);
}

void launch_norm_cast(const float* h, const float* y, int S, const void* gamma, float eps, int T,
                      int H, int dt, void* xo, float* h_out, hipStream_t s) {
  // one token per block for decode-sized batches (more blocks in flight)
  const int tpb = T <= 512 ? 1 : 4;
  const int nb = (T + tpb - 1) / tpb;
  const size_t nlds = static_cast<size_t>(tpb) * H * sizeof(float);
  const bool few = y == nullptr || S <= 8;  // slot loads unrolled to 8 or 16
  auto go = [&](auto wt, auto tp, auto sl) {
    using WT = decltype(wt);
    norm_cast_kernel<WT, decltype(tp)::value, decltype(sl)::value>
        <<<nb, norm_threads<decltype(tp)::value>(), nlds, s>>>(
        h, y, S, static_cast<const WT*>(gamma), eps, T, H, static_cast<WT*>(xo), h_out);
  };
  using I1 = std::integral_constant<int, 1>;
  using I4 = std::integral_constant<int, 4>;
  using S8 = std::integral_constant<int, 8>;
  using S16 = std::integral_constant<int, kNormMaxSlots>;
  if (dt == MOEV_BF16) {
    if (tpb == 1) few ? go(u16{}, I1{}, S8{}) : go(u16{}, I1{}, S16{});
    else few ? go(u16{}, I4{}, S8{}) : go(u16{}, I4{}, S16{});
  } else {
    if (tpb == 1) few ? go(float{}, I1{}, S8{}) : go(float{}, I1{}, S16{});
    else few ? go(float{}, I4{}, S8{}) : go(float{}, I4{}, S16{});
  }
}

void launch_lmhead(const float* h, const void* norm_f, float eps, const void* w_lm, int T, int H,
                   int V, int dt, int32_t* argmax_out, float* max_out, float* logits_out,
                   void* ws, hipStream_t s, const float* y_prev, int S_prev, float* h_out,
                   int out_stride, const VerifyFuse* vf) {
  const size_t xf_bytes = align_up(static_cast<size_t>(T) * H * esize(dt), 256);
  const int nblk = head_blocks(V);
  const size_t part = align_up(static_cast<size_t>(nblk) * T * 4, 256);
  unsigned char* base = static_cast<unsigned char*>(ws);
  void* xf = base;
  float* pmax = reinterpret_cast<float*>(base + xf_bytes);
  int32_t* pidx = reinterpret_cast<int32_t*>(base + xf_bytes + part);
  GemmArgs hd{};
  hd.w0 = w_lm;
  hd.w_group = 0;
  hd.N = V;
  hd.K = H;
  hd.x = xf;
  hd.T = T;
  hd.out = pmax;
  hd.out_idx = pidx;
  hd.logits = logits_out;
  launch_norm_cast(h, y_prev, S_prev, norm_f, eps, T, H, dt, xf, h_out, s);
  if (dt == MOEV_BF16) {
    if (T >= kHeadTileMinTokens) launch_tile_head<u16>(hd, nblk, s);
    else launch_gemm<u16, kHead, kRtHead, kWavesHead>(hd, dim3(nblk), s);
  } else {
    launch_gemm<float, kHead, kRtHead, kWavesHead>(hd, dim3(nblk), s);
  }
  // (the attention step's checks keep it on the fused path: K + 1 <= 16)
  if (vf != nullptr && vf->K + 1 <= kVerifyFuseMaxRows && out_stride == 1 && max_out == nullptr) {
    argmax_verify_kernel<<<vf->B, 64 * (vf->K + 1), 0, s>>>(pmax, pidx, nblk, argmax_out, *vf);
    return;
  }
  argmax_reduce_kernel<<<T, 64, 0, s>>>(pmax, pidx, nblk, T, argmax_out, out_stride, max_out);
  if (vf != nullptr)
    launch_verify(vf->tokens, argmax_out, vf->B, vf->K, vf->n_accept, vf->commit, vf->commit_len,
                  vf->next_last, s);
}

moev_status validate_grouped_ffn(const void* x, const int32_t* sorted_src, const int32_t* offsets,
                                 const float* topk_w, const void* w_gate, const void* w_up,
                                 const void* w_down, int T, int H, int I, int E, int k, int ns,
                                 int dt, const float* y_slots, const void* ws, size_t ws_bytes) {
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  if (moev_status st = check_hid(H)) return st;
  if (moev_status st = check_inter(I)) return st;
  MOEV_REQUIRE(T >= 0, MOEV_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  MOEV_REQUIRE(E >= 1 && E <= 64, MOEV_ERR_UNSUPPORTED, "routed experts E=%d must be in [1, 64]", E);
  MOEV_REQUIRE(k >= 1 && k <= E, MOEV_ERR_UNSUPPORTED, "top-k k=%d must be in [1, E=%d]", k, E);
  MOEV_REQUIRE(ns >= 0 && ns <= 8, MOEV_ERR_UNSUPPORTED, "shared experts ns=%d must be in [0, 8]", ns);
  MOEV_REQUIRE(static_cast<long long>(T) * (k + ns) < (1ll << 31), MOEV_ERR_UNSUPPORTED,
               "T*(k+ns) must be < 2^31");
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(x, "x") && need_ptr(sorted_src, "sorted_src", 4) &&
                 need_ptr(offsets, "group_offsets", 4) && need_ptr(topk_w, "topk_w", 4) &&
                 need_ptr(w_gate, "w_gate") && need_ptr(w_up, "w_up") &&
                 need_ptr(w_down, "w_down") && need_ptr(y_slots, "y_slots"),
             MOEV_ERR_INVALID_ARG);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE,
               "workspace must be non-NULL and 16-byte aligned");
  const size_t need = grouped_ffn_ws_bytes(T, I, k, ns, dt);
  MOEV_REQUIRE(ws_bytes >= need, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
               ws_bytes, need);
  return MOEV_OK;
}

moev_status validate_ffn_stage(const void* in, const int32_t* sorted_src, const int32_t* offsets,
                               const void* w_a, const void* w_b, int T, int H, int I, int E, int k,
                               int ns, int dt, const void* out) {
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  if (moev_status st = check_hid(H)) return st;
  if (moev_status st = check_inter(I)) return st;
  MOEV_REQUIRE(T >= 0, MOEV_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  MOEV_REQUIRE(E >= 1 && E <= 64, MOEV_ERR_UNSUPPORTED, "routed experts E=%d must be in [1, 64]", E);
  MOEV_REQUIRE(k >= 1 && k <= E, MOEV_ERR_UNSUPPORTED, "top-k k=%d must be in [1, E=%d]", k, E);
  MOEV_REQUIRE(ns >= 0 && ns <= 8, MOEV_ERR_UNSUPPORTED, "shared experts ns=%d must be in [0, 8]", ns);
  MOEV_REQUIRE(static_cast<long long>(T) * (k + ns) < (1ll << 31), MOEV_ERR_UNSUPPORTED,
               "T*(k+ns) must be < 2^31");
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(in, "input") && need_ptr(sorted_src, "sorted_src", 4) &&
                 need_ptr(offsets, "group_offsets", 4) && need_ptr(w_a, "weights") &&
                 need_ptr(w_b, "weights/topk_w", 4) && need_ptr(out, "output"),
             MOEV_ERR_INVALID_ARG);
  return MOEV_OK;
}

moev_status validate_lmhead(const float* h, const void* norm_f, const void* w_lm, int T, int H,
                            int V, int dt, const int32_t* argmax_out, const float* max_out,
                            const float* logits_out, const void* ws, size_t ws_bytes) {
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  if (moev_status st = check_hid(H)) return st;
  MOEV_REQUIRE(T >= 0, MOEV_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  MOEV_REQUIRE(V >= 1, MOEV_ERR_INVALID_ARG, "vocabulary V must be >= 1 (got %d)", V);
  if (T == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(h, "h") && opt_ptr(norm_f, "norm_f") && need_ptr(w_lm, "w_lm") &&
                 need_ptr(argmax_out, "argmax_out", 4) && opt_ptr(max_out, "max_out", 4) &&
                 opt_ptr(logits_out, "logits_out", 4),
             MOEV_ERR_INVALID_ARG);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE,
               "workspace must be non-NULL and 16-byte aligned");
  const size_t need = lmhead_ws_bytes(T, H, V, dt);
  MOEV_REQUIRE(ws_bytes >= need, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
               ws_bytes, need);
  return MOEV_OK;
}

}  // namespace moev

extern "C" size_t moe_grouped_ffn_workspace_size(int T, int I, int k, int ns, int dt) {
  if (T < 0 || I < 0 || k < 0 || ns < 0) return 0;
  return moev::grouped_ffn_ws_bytes(T, I, k, ns, dt);
}

extern "C" moev_status moe_grouped_ffn(const void* x, const int32_t* sorted_src,
                                       const int32_t* group_offsets, const float* topk_w,
                                       const void* w_gate, const void* w_up, const void* w_down,
                                       int T, int H, int I, int E, int k, int ns, int dt,
                                       float* y_slots, void* ws, size_t ws_bytes, void* stream) {
  if (moev_status st = moev::validate_grouped_ffn(x, sorted_src, group_offsets, topk_w, w_gate,
                                                  w_up, w_down, T, H, I, E, k, ns, dt, y_slots,
                                                  ws, ws_bytes))
    return st;
  if (T == 0) return MOEV_OK;
  moev::launch_grouped_ffn(x, sorted_src, group_offsets, topk_w, w_gate, w_up, w_down, T, H, I, E,
                           k, ns, dt, y_slots, ws, moev::as_stream(stream));
  return moev::launch_status("moe_grouped_ffn");
}

extern "C" moev_status moe_ffn_gate_up(const void* x, const int32_t* sorted_src,
                                       const int32_t* group_offsets, const void* w_gate,
                                       const void* w_up, int T, int H, int I, int E, int k, int ns,
                                       int dt, void* act, void* stream) {
  if (moev_status st = moev::validate_ffn_stage(x, sorted_src, group_offsets, w_gate, w_up, T, H, I,
                                                E, k, ns, dt, act))
    return st;
  if (T == 0) return MOEV_OK;
  moev::launch_ffn_gate_up(x, sorted_src, group_offsets, w_gate, w_up, T, H, I, E, k, ns, dt, act,
                           moev::as_stream(stream));
  return moev::launch_status("moe_ffn_gate_up");
}

extern "C" moev_status moe_ffn_down(const void* act, const int32_t* sorted_src,
                                    const int32_t* group_offsets, const float* topk_w,
                                    const void* w_down, int T, int H, int I, int E, int k, int ns,
                                    int dt, float* y_slots, void* stream) {
  if (moev_status st = moev::validate_ffn_stage(act, sorted_src, group_offsets, w_down, topk_w, T,
                                                H, I, E, k, ns, dt, y_slots))
    return st;
  if (T == 0) return MOEV_OK;
  moev::launch_ffn_down(act, sorted_src, group_offsets, topk_w, w_down, T, H, I, E, k, ns, dt,
                        y_slots, moev::as_stream(stream));
  return moev::launch_status("moe_ffn_down");
}

extern "C" size_t lmhead_argmax_workspace_size(int T, int H, int V, int dt) {
  if (T < 0 || H < 0 || V < 1) return 0;
  return moev::lmhead_ws_bytes(T, H, V, dt);
}

extern "C" moev_status lmhead_argmax(const float* h, const void* norm_f, float eps,
                                     const void* w_lm, int T, int H, int V, int dt,
                                     int32_t* argmax_out, float* max_out, float* logits_out,
                                     void* ws, size_t ws_bytes, void* stream) {
  if (moev_status st = moev::validate_lmhead(h, norm_f, w_lm, T, H, V, dt, argmax_out, max_out,
                                             logits_out, ws, ws_bytes))
    return st;
  if (T == 0) return MOEV_OK;
  moev::launch_lmhead(h, norm_f, eps, w_lm, T, H, V, dt, argmax_out, max_out, logits_out, ws,
                      moev::as_stream(stream));
  return moev::launch_status("lmhead_argmax");
}

namespace moev {
size_t packed_elems(int G, int N, int K) {
  return static_cast<size_t>(G) * ((static_cast<size_t>(N) + 15) / 16 * 16) * K;
}
}  // namespace moev

extern "C" size_t moev_packed_size(int G, int N, int K, int dt) {
  if (G < 1 || N < 1 || K < 32 || K % 32 != 0 || (dt != MOEV_BF16 && dt != MOEV_F32)) return 0;
  return moev::packed_elems(G, N, K) * (dt == MOEV_BF16 ? 2 : 4);
}

extern "C" moev_status moev_pack_weights(const void* src, void* dst, int G, int N, int K, int dt,
                                         void* stream) {
  using namespace moev;
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  MOEV_REQUIRE(G >= 1 && N >= 1, MOEV_ERR_INVALID_ARG, "need G >= 1 and N >= 1 (G=%d N=%d)", G, N);
  MOEV_REQUIRE(K >= 32 && K % 32 == 0, MOEV_ERR_UNSUPPORTED, "K=%d must be a positive multiple of 32", K);
  MOEV_CHECK(need_ptr(src, "src") && need_ptr(dst, "dst"), MOEV_ERR_INVALID_ARG);
  const long long total = static_cast<long long>(G) * ((N + 15) / 16) * (K / 32) * 64;
  const int blocks = static_cast<int>(min(8192ll, (total + 255) / 256));
  const hipStream_t s = as_stream(stream);
  if (dt == MOEV_BF16)
    pack_kernel<u16><<<blocks, 256, 0, s>>>(static_cast<const u16*>(src), static_cast<u16*>(dst), G, N, K);
  else
    pack_kernel<float><<<blocks, 256, 0, s>>>(static_cast<const float*>(src), static_cast<float*>(dst), G, N, K);
  return launch_status("moev_pack_weights");
}
