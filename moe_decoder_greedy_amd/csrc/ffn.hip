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

#ifndef MOEV_KC
#define MOEV_KC 64
#endif
#ifndef MOEV_KNB
#define MOEV_KNB 3
#endif
#ifndef MOEV_KNBD
#define MOEV_KNBD 3
#endif
constexpr int kKC = MOEV_KC;     // K elements per LDS chunk (multiple of 32)
constexpr int kKB = kKC / 32;    // MFMA K blocks per chunk
constexpr int kNB = MOEV_KNB;    // LDS path: weight ring depth in chunks
constexpr int kNBD = MOEV_KNBD;  // direct path: ring depth in K blocks
constexpr int kFrag = 512;       // elements of one packed 16x32 fragment
#ifndef MOEV_RT_DOWN
#define MOEV_RT_DOWN 1
#endif
#ifndef MOEV_RT_HEAD
#define MOEV_RT_HEAD 2
#endif
#ifndef MOEV_WAVES_HEAD
#define MOEV_WAVES_HEAD 8
#endif
constexpr int kRtDown = MOEV_RT_DOWN;        // 16-row tiles per wave, down projection
constexpr int kRtHead = MOEV_RT_HEAD;        // 16-row tiles per wave, LM head
constexpr int kWavesFfn = 4;                 // wavefronts per workgroup, expert GEMMs
#ifndef MOEV_TILE_MIN_TOKENS
#define MOEV_TILE_MIN_TOKENS 512
#endif
constexpr int kTileMinTokens = MOEV_TILE_MIN_TOKENS;  // larger batches use the tile schedule
constexpr int kWavesHead = MOEV_WAVES_HEAD;  // wavefronts per workgroup, LM head

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
  int S, k, P, T;           // slots, routed slots, pairs, tokens
  int n_first;              // the last n_first groups (the shared experts, which
                            // hold every token) are dispatched first
  const float* topk_w;      // [T, k] (down)
  void* out;                // gate/up: act [P, N] WT; down: y [P, N] fp32; head: pmax
  int32_t* out_idx;         // head: partial arg max [blocks, T]
  float* logits;            // head: optional logits [T, N]
};

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

// Row of the operand matrix that token row `row` of this pass reads.
template <int MODE>
__device__ __forceinline__ long long operand_row(const GemmArgs& a, int off, int m0, int row) {
  if (MODE == kGateUp) return clampi(a.sorted_src[off + m0 + row], 0, a.P - 1) / a.S;
  if (MODE == kDown) return off + m0 + row;
  return m0 + row;
}

// Epilogue of one pass: lane (r16, q) holds rows rowbase[rt] + 4q + v of
// token column j*16 + r16.
template <typename WT, int MODE, int RT, int MT, int NTX, int W>
__device__ __forceinline__ void epilogue(const GemmArgs& a, unsigned char* __restrict__ lds,
                                         const f32x4 (&acc)[RT][NTX], int off, int m0, int mp,
                                         const int (&rowbase)[RT]) {
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
        for (int v = 0; v < 4; ++v) o[v] = gv[v] / (1.0f + expf(-gv[v])) * uv[v];
        store4<WT>(act + static_cast<long long>(off + m0 + m) * a.N + n, o);
      }
    }
  } else if (MODE == kDown) {
    float* y = static_cast<float*>(a.out);
#pragma unroll
    for (int j = 0; j < NTX; ++j) {
      const int m = j * 16 + r16;
      if (m < mp) {
        const int p = clampi(a.sorted_src[off + m0 + m], 0, a.P - 1);
        const int t = p / a.S;
        const int slot = p - t * a.S;
        const float wgt = slot < a.k ? a.topk_w[static_cast<long long>(t) * a.k + slot] : 1.0f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          f32x4 o = acc[rt][j];
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] *= wgt;
          store4<float>(y + static_cast<long long>(p) * a.N + rowbase[rt] + 4 * q, o);
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
      const long long o = static_cast<long long>(blockIdx.x) * a.T + m0 + tid;
      static_cast<float*>(a.out)[o] = best;
      a.out_idx[o] = bi;
    }
  }
}

// Direct pass (mp <= 16 * NTX <= 32): both fragments come from global memory
// through one register ring kNBD K blocks deep; no LDS, no barriers.  Token
// rows past mp read row 0 of the pass and are dropped by the epilogue.
template <typename WT, int MODE, int RT, int MT, int NTX, int W>
__device__ __forceinline__ void gemm_pass_direct(const GemmArgs& a, unsigned char* __restrict__ lds,
                                                 int off, int m0, int mp,
                                                 const WT* const (&wp)[RT],
                                                 const int (&rowbase)[RT]) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int K = a.K;
  const int nkb = K / 32;
  const WT* __restrict__ xsrc = static_cast<const WT*>(a.x);
  const WT* xp[NTX];
#pragma unroll
  for (int j = 0; j < NTX; ++j) {
    const int m = j * 16 + r16;
    xp[j] = xsrc + operand_row<MODE>(a, off, m0, m < mp ? m : 0) * K + q * 8;
  }
  f32x4 acc[RT][NTX];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NTX; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Frag<WT> rw[kNBD][RT], rx[kNBD][NTX];
#pragma unroll
  for (int u = 0; u < kNBD; ++u)
    if (u < nkb) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) rw[u][rt].load(wp[rt] + u * kFrag);
#pragma unroll
      for (int j = 0; j < NTX; ++j) rx[u][j].load(xp[j] + u * 32);
    }
  for (int kb0 = 0; kb0 < nkb; kb0 += kNBD) {
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
  epilogue<WT, MODE, RT, MT, NTX, W>(a, lds, acc, off, m0, mp, rowbase);
}

// LDS-staged pass: mt = ceil(mp / 16) <= NTX column tiles.  NTX is a
// compile-time tile count, so the K loop carries no per-tile predicates;
// tiles past mt multiply LDS rows that the staging loop zero-filled and are
// dropped by the epilogue.
template <typename WT, int MODE, int RT, int MT, int NTX, int W>
__device__ __forceinline__ void gemm_pass_lds(const GemmArgs& a, unsigned char* __restrict__ lds,
                                              int off, int m0, int mp,
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
    src[s] = (v < kVecs && row < mp) ? xsrc + operand_row<MODE>(a, off, m0, row) * K + cv * C::kEpv
                                     : nullptr;
  }
  uint4 stage[kStage];
#pragma unroll
  for (int s = 0; s < kStage; ++s)
    stage[s] = src[s] ? *reinterpret_cast<const uint4*>(src[s]) : make_uint4(0, 0, 0, 0);

  f32x4 acc[RT][NTX];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < NTX; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  Frag<WT> ring[kNB][RT][kKB];
#pragma unroll
  for (int u = 0; u < kNB; ++u)
    if (u < nchunks)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int kk = 0; kk < kKB; ++kk) ring[u][rt][kk].load(wp[rt] + (u * kKB + kk) * kFrag);

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
        if (c + kNB < nchunks) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kk = 0; kk < kKB; ++kk)
              ring[u][rt][kk].load(wp[rt] + ((c + kNB) * kKB + kk) * kFrag);
        }
      }
    }
  }
  epilogue<WT, MODE, RT, MT, NTX, W>(a, lds, acc, off, m0, mp, rowbase);
}

template <typename WT, int MODE, int RT, int MT, int W>
__global__ __launch_bounds__(W * 64) void stream_gemm(GemmArgs a) {
  using C = Cfg<WT, MT>;
  constexpr int NT = C::kTiles;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  int g = 0, off = 0, M;
  if (MODE == kHead) {
    M = a.T;
  } else {
    const int G = gridDim.y;
    g = static_cast<int>(blockIdx.y) < a.n_first ? G - a.n_first + blockIdx.y : blockIdx.y - a.n_first;
    off = clampi(a.offsets[g], 0, a.P);
    M = clampi(a.offsets[g + 1], off, a.P) - off;
  }
  if (M <= 0) return;

  const WT* __restrict__ w0 = static_cast<const WT*>(a.w0);
  const WT* __restrict__ w1 = static_cast<const WT*>(a.w1);
  const int nkb = a.K / 32;
  const int ntiles = (a.N + 15) / 16;

  // this wave's weight tiles; lane pointer = its 16 bytes of the first fragment
  const WT* wp[RT];
  int rowbase[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rb = (MODE == kGateUp) ? blockIdx.x * (16 * W) + wave * 16
                                     : blockIdx.x * (16 * RT * W) + wave * (16 * RT) + rt * 16;
    rowbase[rt] = rb;
    const int tile = min(rb / 16, ntiles - 1);
    const WT* base = (MODE == kGateUp && rt == 1) ? w1 : w0;
    wp[rt] = base + static_cast<long long>(g) * a.w_group +
             static_cast<long long>(tile) * nkb * kFrag + lane * 8;
  }

  for (int m0 = 0; m0 < M; m0 += MT) {
    const int mp = min(MT, M - m0);
    // the branches are uniform across the workgroup
    if (mp <= 16) {
      gemm_pass_direct<WT, MODE, RT, MT, 1, W>(a, lds, off, m0, mp, wp, rowbase);
    } else if (mp <= 32) {
      gemm_pass_direct<WT, MODE, RT, MT, 2, W>(a, lds, off, m0, mp, wp, rowbase);
    } else if constexpr (NT >= 4) {
      if (mp <= 64 || NT == 4)
        gemm_pass_lds<WT, MODE, RT, MT, 4, W>(a, lds, off, m0, mp, wp, rowbase);
      else
        gemm_pass_lds<WT, MODE, RT, MT, NT, W>(a, lds, off, m0, mp, wp, rowbase);
    }
  }
}

// ---------------------------------------------------------------------------
// Tile schedule for large groups (prefill-sized batches).
//
// One workgroup computes one (group, column tile, 128-token tile): 4
// wavefronts x 4 weight tiles of 16 rows (gate/up: 2 gate + the same 2 up
// tiles, i.e. 32 intermediate columns per wave, 128 per workgroup; down: 64
// hidden rows per wave, 256 per workgroup) against 8 token tiles.  Weight
// fragments come straight from the packed layout into a register ring; the
// token rows go through a double-buffered LDS chunk (one barrier per 64-wide
// K chunk), and the next chunk's rows are fetched into registers while the
// current one is multiplied.  Tiles of one (group, column tile) are
// consecutive in the tile order and the order is laid out so that consecutive
// tiles land on the same XCD: the workgroups sharing a weight slab run side
// by side and read it through one L2.
// Accumulation is the same single fp32 chain over K blocks in order with the
// same MFMA as the streaming schedule, so results are bitwise identical.
constexpr int kTileTok = 128;                 // tokens per tile
constexpr int kTileRt = 4;                    // 16-row weight tiles per wave
constexpr int kTileNT = kTileTok / 16;        // token tiles per wave
constexpr int kTileThreads = 256;
constexpr int kTileNB = 4;                    // weight ring depth, in chunks (even)
constexpr int kXcds = 8;

template <int MODE> constexpr int tile_cols() { return MODE == kGateUp ? 128 : 256; }

template <typename WT, int MODE>
__global__ __launch_bounds__(kTileThreads) void tile_gemm(GemmArgs a, int n_ctiles, int G) {
  using C = Cfg<WT, kTileTok>;
  constexpr int kVecs = kTileTok * C::kVecPerRow;             // 16-B vectors per chunk
  constexpr int kStage = kVecs / kTileThreads;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][kTileTok * C::kRowBytes];
  __shared__ int tile_info[3];  // group, column tile, token tile (-1: no work)

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;

  // XCD-aware tile index: hardware deals consecutive block ids round-robin
  // over the XCDs, so tile = xcd * (grid / 8) + (bid / 8) keeps a run of
  // consecutive tiles on one XCD.
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int tile = (bid % kXcds) * (nb / kXcds) + bid / kXcds;
  if (tid == 0) {
    int run = 0, g = -1, ct = 0, mt = 0;
    for (int gg = 0; gg < G && g < 0; ++gg) {
      const int M = max(0, min(a.offsets[gg + 1], a.P) - max(min(a.offsets[gg], a.P), 0));
      const int mtiles = (M + kTileTok - 1) / kTileTok;
      const int n = mtiles * n_ctiles;
      if (tile < run + n) {
        g = gg;
        ct = (tile - run) / mtiles;
        mt = (tile - run) - ct * mtiles;
      }
      run += n;
    }
    tile_info[0] = g;
    tile_info[1] = ct;
    tile_info[2] = mt;
  }
  __syncthreads();
  const int g = tile_info[0];
  if (g < 0) return;
  const int ct = tile_info[1];
  const int off = clampi(a.offsets[g], 0, a.P);
  const int M = clampi(a.offsets[g + 1], off, a.P) - off;
  const int m0 = tile_info[2] * kTileTok;
  const int mp = min(kTileTok, M - m0);

  const WT* __restrict__ w0 = static_cast<const WT*>(a.w0);
  const WT* __restrict__ w1 = static_cast<const WT*>(a.w1);
  const WT* __restrict__ xsrc = static_cast<const WT*>(a.x);
  const int K = a.K;
  const int nkb = K / 32;
  const int nchunks = K / kKC;

  // this wave's weight tiles and their first output row
  const WT* wp[kTileRt];
  int rowbase[kTileRt];
#pragma unroll
  for (int rt = 0; rt < kTileRt; ++rt) {
    int rb;
    const WT* base;
    if (MODE == kGateUp) {  // tiles 0,1: gate columns c0, c0+16; tiles 2,3: up, same columns
      rb = ct * tile_cols<MODE>() + wave * 32 + (rt & 1) * 16;
      base = rt < 2 ? w0 : w1;
    } else {
      rb = ct * tile_cols<MODE>() + wave * 64 + rt * 16;
      base = w0;
    }
    rowbase[rt] = rb;
    wp[rt] = base + static_cast<long long>(g) * a.w_group + static_cast<long long>(rb / 16) * nkb * kFrag +
             lane * 8;
  }

  // token rows of this thread's staging vectors (nullptr: zero-fill)
  const WT* src[kStage];
#pragma unroll
  for (int s = 0; s < kStage; ++s) {
    const int v = tid + s * kTileThreads;
    const int row = v / C::kVecPerRow;
    const int cv = v - row * C::kVecPerRow;
    src[s] = row < mp ? xsrc + operand_row<MODE>(a, off, m0, row) * K + cv * C::kEpv : nullptr;
  }
  auto fetch = [&](uint4 (&st)[kStage], int c) {
#pragma unroll
    for (int s = 0; s < kStage; ++s)
      st[s] = src[s] ? *reinterpret_cast<const uint4*>(src[s] + c * kKC) : make_uint4(0, 0, 0, 0);
  };
  auto put = [&](const uint4 (&st)[kStage], unsigned char* buf) {
#pragma unroll
    for (int s = 0; s < kStage; ++s) {
      const int v = tid + s * kTileThreads;
      const int row = v / C::kVecPerRow;
      const int cv = v - row * C::kVecPerRow;
      *reinterpret_cast<uint4*>(buf + row * C::kRowBytes + cv * 16) = st[s];
    }
  };

  f32x4 acc[kTileRt][kTileNT];
#pragma unroll
  for (int rt = 0; rt < kTileRt; ++rt)
#pragma unroll
    for (int j = 0; j < kTileNT; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Pipeline (loads complete in issue order, so every wait also covers the
  // loads issued before it): in iteration c the token rows of chunk c+2 and
  // the weights of chunk c+kTileNB are requested, and the rows of chunk c+1
  // (requested an iteration earlier, ahead of the weights of chunk c+kTileNB-1)
  // are written to the other LDS buffer; one barrier per chunk.
  uint4 st0[kStage], st1[kStage];
  fetch(st0, 0);
  Frag<WT> ring[kTileNB][kTileRt][kKB];
#pragma unroll
  for (int u = 0; u < kTileNB; ++u)
    if (u < nchunks)
#pragma unroll
      for (int rt = 0; rt < kTileRt; ++rt)
#pragma unroll
        for (int kk = 0; kk < kKB; ++kk) ring[u][rt][kk].load(wp[rt] + (u * kKB + kk) * kFrag);
  if (nchunks > 1) fetch(st1, 1);
  put(st0, lds[0]);
  __syncthreads();

  // kTileNB is a multiple of 2, so u and c share parity and the stage sets
  // can be named statically
  for (int c0 = 0; c0 < nchunks; c0 += kTileNB) {
#pragma unroll
    for (int u = 0; u < kTileNB; ++u) {
      const int c = c0 + u;
      if (c < nchunks) {
        uint4 (&st_next)[kStage] = (u & 1) ? st0 : st1;   // holds chunk c+1
        uint4 (&st_free)[kStage] = (u & 1) ? st1 : st0;   // held chunk c, now in LDS
        if (c + 2 < nchunks) fetch(st_free, c + 2);
        const unsigned char* buf = lds[c & 1];
#pragma unroll
        for (int kk = 0; kk < kKB; ++kk) {
          Frag<WT> b[kTileNT];
#pragma unroll
          for (int j = 0; j < kTileNT; ++j)
            b[j].load(reinterpret_cast<const WT*>(buf + (j * 16 + r16) * C::kRowBytes) + kk * 32 + q * 8);
#pragma unroll
          for (int j = 0; j < kTileNT; ++j)
#pragma unroll
            for (int rt = 0; rt < kTileRt; ++rt) acc[rt][j] = mma(ring[u][rt][kk], b[j], acc[rt][j]);
        }
        if (c + kTileNB < nchunks) {
#pragma unroll
          for (int rt = 0; rt < kTileRt; ++rt)
#pragma unroll
            for (int kk = 0; kk < kKB; ++kk)
              ring[u][rt][kk].load(wp[rt] + ((c + kTileNB) * kKB + kk) * kFrag);
        }
        if (c + 1 < nchunks) put(st_next, lds[(c + 1) & 1]);
        __syncthreads();
      }
    }
  }

  // epilogue: lane (r16, q) holds rows rowbase[rt] + 4q + v of token column j*16 + r16
  if (MODE == kGateUp) {
    WT* act = static_cast<WT*>(a.out);
#pragma unroll
    for (int j = 0; j < kTileNT; ++j) {
      const int m = j * 16 + r16;
      if (m < mp) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 gv = acc[h][j], uv = acc[2 + h][j];
          f32x4 o;
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = gv[v] / (1.0f + expf(-gv[v])) * uv[v];
          store4<WT>(act + static_cast<long long>(off + m0 + m) * a.N + rowbase[h] + 4 * q, o);
        }
      }
    }
  } else {
    float* y = static_cast<float*>(a.out);
#pragma unroll
    for (int j = 0; j < kTileNT; ++j) {
      const int m = j * 16 + r16;
      if (m < mp) {
        const int p = clampi(a.sorted_src[off + m0 + m], 0, a.P - 1);
        const int t = p / a.S;
        const int slot = p - t * a.S;
        const float wgt = slot < a.k ? a.topk_w[static_cast<long long>(t) * a.k + slot] : 1.0f;
#pragma unroll
        for (int rt = 0; rt < kTileRt; ++rt) {
          f32x4 o = acc[rt][j];
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] *= wgt;
          store4<float>(y + static_cast<long long>(p) * a.N + rowbase[rt] + 4 * q, o);
        }
      }
    }
  }
}

// Upper bound of the tile count (groups are only known on the device): every
// group contributes at most ceil(M_g / 128) <= M_g / 128 + 1 token tiles.
int tile_grid(int T, int k, int ns, int E, int n_ctiles) {
  const long long routed = (static_cast<long long>(T) * k + kTileTok - 1) / kTileTok + E;
  const long long shared = static_cast<long long>(ns) * ((T + kTileTok - 1) / kTileTok);
  long long n = (routed + shared) * n_ctiles;
  n = (n + kXcds - 1) / kXcds * kXcds;
  return static_cast<int>(n);
}

template <typename WT, int MODE>
void launch_tile(const GemmArgs& args, int n_ctiles, int G, int E, int k, int ns, hipStream_t s) {
  const int grid = tile_grid(args.T, k, ns, E, n_ctiles);
  tile_gemm<WT, MODE><<<grid, kTileThreads, 0, s>>>(args, n_ctiles, G);
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

// Final RMSNorm of the head input, rounded to the operand type: one block of
// 256 threads per 4 tokens.  With y (the last layer's expert slots) the
// residual add happens first, in the same slot order as the combine kernel,
// every slot load of a thread issued before the sum.
constexpr int kNormTPB = 4;
constexpr int kNormMaxSlots = 16;

template <typename WT>
__global__ __launch_bounds__(256) void norm_cast_kernel(const float* __restrict__ h,
                                                        const float* __restrict__ y, int S,
                                                        const WT* __restrict__ gamma, float eps,
                                                        int T, int H, WT* __restrict__ xo) {
  extern __shared__ float hs[];   // [kNormTPB][H]
  const int t0 = blockIdx.x * kNormTPB;
  const int nt = min(kNormTPB, T - t0);
  const int h4 = H / 4;
  for (int f = threadIdx.x; f < nt * h4; f += 256) {
    const int tt = f / h4;
    const int i = (f - tt * h4) * 4;
    const long long t = t0 + tt;
    float4 v = *reinterpret_cast<const float4*>(h + t * H + i);
    if (y != nullptr) {
      const float4* ys = reinterpret_cast<const float4*>(y + t * S * H + i);
      float4 sv[kNormMaxSlots];
#pragma unroll
      for (int sl = 0; sl < kNormMaxSlots; ++sl)
        if (sl < S) sv[sl] = ys[static_cast<long long>(sl) * h4];
      float4 acc = sv[0];
#pragma unroll
      for (int sl = 1; sl < kNormMaxSlots; ++sl)
        if (sl < S) {
          acc.x += sv[sl].x;
          acc.y += sv[sl].y;
          acc.z += sv[sl].z;
          acc.w += sv[sl].w;
        }
      v = make_float4(v.x + acc.x, v.y + acc.y, v.z + acc.z, v.w + acc.w);
    }
    *reinterpret_cast<float4*>(hs + tt * H + i) = v;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (wave >= nt) return;
  const float* hr = hs + wave * H;
  float ss = 0.f;
  for (int i = lane * 4; i < H; i += 256) {
    const float4 v = *reinterpret_cast<const float4*>(hr + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = lane63(wave_sum_lane63(ss));
  const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
  for (int i = lane * 4; i < H; i += 256) {
    const float4 v = *reinterpret_cast<const float4*>(hr + i);
    f32x4 o;
    o[0] = v.x * r * (gamma ? to_f32<WT>(gamma[i + 0]) : 1.f);
    o[1] = v.y * r * (gamma ? to_f32<WT>(gamma[i + 1]) : 1.f);
    o[2] = v.z * r * (gamma ? to_f32<WT>(gamma[i + 2]) : 1.f);
    o[3] = v.w * r * (gamma ? to_f32<WT>(gamma[i + 3]) : 1.f);
    store4<WT>(xo + static_cast<long long>(t0 + wave) * H + i, o);
  }
}

// Second pass of the blocked arg max: one wavefront per token.
__global__ __launch_bounds__(64) void argmax_reduce_kernel(const float* __restrict__ pmax,
                                                           const int32_t* __restrict__ pidx,
                                                           int nblk, int T,
                                                           int32_t* __restrict__ argmax_out,
                                                           float* __restrict__ max_out) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int b = lane; b < nblk; b += 64) {
    const float v = pmax[static_cast<long long>(b) * T + t];
    const int i = pidx[static_cast<long long>(b) * T + t];
    if (better(v, i, best, bi)) { best = v; bi = i; }
  }
  wave_argmax(best, bi);
  if (lane == 0) {
    argmax_out[t] = bi;
    if (max_out) max_out[t] = best;
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

void launch_grouped_ffn(const void* x, const int32_t* sorted_src, const int32_t* offsets,
                        const float* topk_w, const void* w_gate, const void* w_up,
                        const void* w_down, int T, int H, int I, int E, int k, int ns, int dt,
                        float* y_slots, void* ws, hipStream_t s) {
  launch_ffn_gate_up(x, sorted_src, offsets, w_gate, w_up, T, H, I, E, k, ns, dt, ws, s);
  launch_ffn_down(ws, sorted_src, offsets, topk_w, w_down, T, H, I, E, k, ns, dt, y_slots, s);
}

void launch_lmhead(const float* h, const void* norm_f, float eps, const void* w_lm, int T, int H,
                   int V, int dt, int32_t* argmax_out, float* max_out, float* logits_out,
                   void* ws, hipStream_t s, const float* y_prev, int S_prev) {
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
  const int nb = (T + kNormTPB - 1) / kNormTPB;
  const size_t nlds = static_cast<size_t>(kNormTPB) * H * sizeof(float);
  if (dt == MOEV_BF16) {
    norm_cast_kernel<u16><<<nb, 256, nlds, s>>>(h, y_prev, S_prev, static_cast<const u16*>(norm_f), eps,
                                              T, H, static_cast<u16*>(xf));
    launch_gemm<u16, kHead, kRtHead, kWavesHead>(hd, dim3(nblk), s);
  } else {
    norm_cast_kernel<float><<<nb, 256, nlds, s>>>(h, y_prev, S_prev, static_cast<const float*>(norm_f),
                                                eps, T, H, static_cast<float*>(xf));
    launch_gemm<float, kHead, kRtHead, kWavesHead>(hd, dim3(nblk), s);
  }
  argmax_reduce_kernel<<<T, 64, 0, s>>>(pmax, pidx, nblk, T, argmax_out, max_out);
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
