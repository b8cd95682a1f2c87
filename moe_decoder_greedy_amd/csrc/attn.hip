// Decode attention: each sequence's verify rows (its last committed token and
// K drafts, run as one pass by the FastMTP verifier -- "The speed comes from
// three layers working together", Jina-OCR-v1 explainer on kg.zhiyong.dev)
// attend causally to the sequence's cached prefix and to each other.  The
// pages do not describe the decoder's attention; this is plain multi-head
// attention with scale 1/sqrt(head width) and no positional rotation: row i
// of sequence b, at position pos[b] + i, sees positions 0 .. pos[b] + i.
//
// The caches are head-major, [B, n_heads, max_len, D]: a (sequence, head)'s
// keys and values are each one contiguous block, read front to back.
// kAttnSplits workgroups per (sequence, head), each of kAttnWaves wavefronts:
// 64-position chunk c of the positions the sequence's last row can see goes
// to split (c / kAttnWaves) mod kAttnSplits and, there, to wave
// c mod kAttnWaves.  A row's visible chunks, the order a wave takes them in
// and both merge orders (waves in a split, then splits) therefore do not
// depend on the number of rows in the pass (chunks a row cannot see leave its
// state unchanged).  Each split writes its unnormalised softmax state
// (maximum, sum, weighted values) to a workspace; attn_merge_kernel combines
// the splits (in the verify step the last split of a (sequence, head) to
// finish does, see attn_decode_kernel's FUSE).  Splitting shortens each
// workgroup's chain of dependent chunk loads, which bounds the kernel, and
// spreads the work over more CUs.  Per
// chunk: four lanes share a key row, each multiplying its D/4 adjacent
// columns by every verify row's query (staged in LDS) and the four summing
// their parts in a fixed order, so a load instruction covers 16 rows in
// 64-byte pieces (one lane per row would touch 64 lines per instruction, and
// more lanes per row cost more shuffles than they save); lane l then takes
// position c0 + l's scores (rows masked causally), each row's chunk maximum
// updates that row's running maximum of an online softmax, and the values
// are accumulated position by position in order, each lane holding D/64
// adjacent output columns of every row, so every key and value row is read
// once per workgroup.  At the end the waves' partial (maximum, sum, output) triples are
// merged in wave order through LDS.  All arithmetic is fp32; a row's result
// depends only on its own query and cache.
#include "launch.h"

namespace moev {
namespace {

constexpr int kAttnMaxRows = 16;   // verify rows per sequence

// N consecutive cache elements as fp32, in one load where the width allows
template <typename WT, int N> __device__ __forceinline__ void ldn(const WT* p, float (&v)[N]) {
  if constexpr (sizeof(WT) == 2 && N == 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_to_f32(w[e] & 0xFFFF);
      v[2 * e + 1] = bf16_to_f32(w[e] >> 16);
    }
  } else if constexpr (sizeof(WT) == 2 && N == 2) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    v[0] = bf16_to_f32(u & 0xFFFF);
    v[1] = bf16_to_f32(u >> 16);
  } else if constexpr (sizeof(WT) == 2 && N == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = bf16_to_f32(u.x & 0xFFFF);
    v[1] = bf16_to_f32(u.x >> 16);
    v[2] = bf16_to_f32(u.y & 0xFFFF);
    v[3] = bf16_to_f32(u.y >> 16);
  } else if constexpr (sizeof(WT) == 4 && N == 2) {
    const float2 u = *reinterpret_cast<const float2*>(p);
    v[0] = u.x;
    v[1] = u.y;
  } else if constexpr (sizeof(WT) == 4 && N == 4) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = to_f32<WT>(p[e]);
  }
}

constexpr int kAttnWaves = 4;   // wavefronts per workgroup
constexpr int kAttnSplits = 3;  // workgroups per (sequence, head)

// Row r, column c of one (sequence, head)'s output: its splits' states
// (po: [kAttnSplits, rows, D] weighted values, pml: [kAttnSplits, rows, 2]
// maximum and sum) merged in split order and normalised.  LD reads one
// state value.  Both merge paths use this one expression.
template <typename LD>
__device__ __forceinline__ float merge_splits(const float* po, const float* pml, int rows, int D, int r, int c,
                                              LD ld) {
#pragma clang fp contract(off)
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kAttnSplits; ++sp) M = fmaxf(M, ld(pml + (sp * rows + r) * 2));
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int sp = 0; sp < kAttnSplits; ++sp) {
    const float m = ld(pml + (sp * rows + r) * 2);
    const float f = m == -INFINITY ? 0.f : expf(m - M);
    L = fmaf(ld(pml + (sp * rows + r) * 2 + 1), f, L);
    O = fmaf(ld(po + (static_cast<long long>(sp) * rows + r) * D + c), f, O);
  }
  return O / L;
}

// Device-coherent (agent-scope) loads and stores of split states: they
// bypass a stale copy in another XCD's L2, so a state written by one
// workgroup is read by another within one launch without cache maintenance.
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// part: the splits' states, [B, n_heads, kAttnSplits, rows, D] weighted
// values, then [B, n_heads, kAttnSplits, rows, 2] (maximum, sum)
// FUSE: each split writes its state with device-coherent stores, waits for
// them, then counts itself in cnt[b, h] (an agent-scope atomic, no waiting on
// anyone); the split that counts last merges the three states, read back in
// split order with device-coherent loads, into out [B*rows, H] (rounded to
// WT once) and resets the count.  Which split merges does not change a bit.
template <typename WT, int D, int R, bool FUSE>
__global__ __launch_bounds__(kWave * kAttnWaves) void attn_decode_kernel(
    const float* __restrict__ q, const WT* __restrict__ kc, const WT* __restrict__ vc,
    const int32_t* __restrict__ pos, int rows, int max_len, int H, float scale, float* __restrict__ part,
    int* __restrict__ cnt, WT* __restrict__ out) {
  // Every fused multiply-add below is written out and no other is formed, so
  // the instantiations for different row counts round identically (the
  // compiler may otherwise fuse a*b + c*d either way round).
#pragma clang fp contract(off)
  // value walk: a value row is read as D / kEpl 16-byte pieces (kLpk lanes);
  // the kNg lane groups of a wave take every kNg-th position of a chunk
  constexpr int kEpl = 16 / static_cast<int>(sizeof(WT));  // elements per 16-byte load
  constexpr int kLpk = D / kEpl;                           // lanes per value row
  constexpr int kNg = kWave / kLpk;                        // position groups
  static_assert(kLpk * kNg == kWave && kLpk >= 1, "head width");
  // LDS: queries [R][D] and per-wave softmax weights [waves][R][64] during
  // the walk; the same space then holds the per-wave outputs [waves][R][D]
  constexpr int kWalk = R * D + kAttnWaves * R * kWave;
  constexpr int kMerge = kAttnWaves * R * D;
  __shared__ float smem[(kWalk > kMerge ? kWalk : kMerge) + 2 * kAttnWaves * R];
  float (*q_s)[D] = reinterpret_cast<float (*)[D]>(smem);
  float (*p_s)[R][kWave] = reinterpret_cast<float (*)[R][kWave]>(smem + R * D);
  float (*o_s)[R][D] = reinterpret_cast<float (*)[R][D]>(smem);
  float (*m_s)[R] = reinterpret_cast<float (*)[R]>(smem + (kWalk > kMerge ? kWalk : kMerge));
  float (*l_s)[R] = m_s + kAttnWaves;
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col0 = h * D;
  for (int i = threadIdx.x; i < R * D; i += blockDim.x) {
    const int r = i / D, c = i - r * D;
    q_s[r][c] = r < rows ? q[(static_cast<long long>(b) * rows + r) * H + col0 + c] * scale : 0.f;
  }
  __syncthreads();

  const int p0 = min(max(pos[b], 0), max_len - rows);  // row r sees positions 0 .. p0 + r
  const int n_all = p0 + rows;
  const int hi = n_all;
  // head-major caches: this (sequence, head)'s rows are one contiguous
  // [max_len, D] block
  const long long blk = (static_cast<long long>(b) * gridDim.y + h) * max_len * D;
  const WT* kb = kc + blk;
  const WT* vb = vc + blk;
  const int vg = lane / kLpk;           // this lane's position group
  const int vc0 = (lane % kLpk) * kEpl;  // and its columns vc0 .. vc0 + kEpl - 1
  // key walk: kKL lanes per key row, each with kKC adjacent columns
  constexpr int kKL = 4, kKC = D / kKL;
  static_assert(kKC % kEpl == 0, "whole loads per key part");
  const int kg = lane / kKL, kc0 = (lane % kKL) * kKC;
  float m_run[R], l_run[R], o[R][kEpl];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) o[r][e] = 0.f;
  }

  const int split = blockIdx.z;
  for (int c0 = (split * kAttnWaves + wave) * kWave; c0 < hi; c0 += kAttnSplits * kAttnWaves * kWave) {
    // scores: kKL lanes per key row, kKC columns each; position jj = it *
    // (64 / kKL) + lane / kKL of the chunk.  The lanes' parts are summed in a
    // fixed order (pairs, then the pair sums) and the first lane files them;
    // positions past hi read the chunk's first row and are masked below
#pragma unroll
    for (int it = 0; it < kKL; ++it) {
      const int jj = it * (kWave / kKL) + kg;
      const int jr = c0 + jj < hi ? c0 + jj : c0;
      float kv[kKC];
#pragma unroll
      for (int c = 0; c < kKC; c += kEpl) {
        float t[kEpl];
        ldn<WT, kEpl>(kb + static_cast<long long>(jr) * D + kc0 + c, t);
#pragma unroll
        for (int e = 0; e < kEpl; ++e) kv[c + e] = t[e];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < kKC; ++e) part = fmaf(q_s[r][kc0 + e], kv[e], part);
        part += dpp_mov<0xb1>(part);  // quad_perm [1,0,3,2]
        part += dpp_mov<0x4e>(part);  // quad_perm [2,3,0,1]
        if (lane % kKL == 0) p_s[wave][r][jj] = part;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int j = c0 + lane;
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = p_s[wave][r][lane];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool vis = j < hi && j <= p0 + r && r < rows;
      const float sv = vis ? s[r] : -INFINITY;
      const float m_new = fmaxf(m_run[r], wave_max(sv));
      // m_new = -inf: nothing of this row visible yet (a row sees fewer
      // positions than the last one); keep its state unchanged
      const float corr = m_new == -INFINITY ? 1.f : expf(m_run[r] - m_new);
      const float pv = vis ? expf(sv - m_new) : 0.f;
      l_run[r] = fmaf(l_run[r], corr, wave_sum(pv));
#pragma unroll
      for (int e = 0; e < kEpl; ++e) o[r][e] *= corr;
      m_run[r] = m_new;
      p_s[wave][r][lane] = pv;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // position jj = it * kNg + vg of the chunk; positions past hi have
    // weight 0 and read the chunk's first row instead
#pragma unroll
    for (int it = 0; it < kWave / kNg; ++it) {
      const int jj = it * kNg + vg;
      const int jr = c0 + jj < hi ? c0 + jj : c0;
      float vv[kEpl];
      ldn<WT, kEpl>(vb + static_cast<long long>(jr) * D + vc0, vv);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float pj = p_s[wave][r][jj];
#pragma unroll
        for (int e = 0; e < kEpl; ++e) o[r][e] = fmaf(pj, vv[e], o[r][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();  // p_s is rewritten by the next chunk
  }

  // merge the waves' partial softmax states, in wave order (every wave is
  // done with the queries and weights before the space is reused)
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (lane == 0) {
      m_s[wave][r] = m_run[r];
      l_s[wave][r] = l_run[r];
    }
    // add the position groups' partial outputs (same columns kLpk lanes apart)
#pragma unroll
    for (int e = 0; e < kEpl; ++e) {
      float v = o[r][e];
#pragma unroll
      for (int m = kLpk; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
      if (vg == 0) o_s[wave][r][vc0 + e] = v;
    }
  }
  __syncthreads();
  // this split's state, unnormalised (maximum -inf, sum 0 when the split
  // holds nothing the row can see)
  const long long slot = (static_cast<long long>(b) * gridDim.y + h) * kAttnSplits + split;
  float* po = part + slot * rows * D;
  float* pml = part + static_cast<long long>(gridDim.x) * gridDim.y * kAttnSplits * rows * D + slot * rows * 2;
  for (int i = threadIdx.x; i < rows * D; i += blockDim.x) {
    const int r = i / D, c = i - r * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, m_s[w][r]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = m_s[w][r] == -INFINITY ? 0.f : expf(m_s[w][r] - M);
      L = fmaf(l_s[w][r], f, L);
      O = fmaf(o_s[w][r][c], f, O);
    }
    if constexpr (FUSE) {
      st_agent(po + r * D + c, O);
      if (c == 0) {
        st_agent(pml + 2 * r, M);
        st_agent(pml + 2 * r + 1, L);
      }
    } else {
      po[r * D + c] = O;
      if (c == 0) {
        pml[2 * r] = M;
        pml[2 * r + 1] = L;
      }
    }
  }
  if constexpr (FUSE) {
    // Ordering, stated for the hardware rather than through C++ fences (an
    // agent-scope release or acquire fence would write back or invalidate
    // the whole L2 of the XCD): (1) the state stores above are agent-scope
    // atomic stores, written through to the device's coherence point; (2)
    // s_waitcnt(0) returns only once every one of them is acknowledged, and
    // the barrier makes that hold for all threads before (3) thread 0's
    // atomic add, which is performed at the coherence point too; (4) the
    // merging split issues its agent-scope loads only after its own add has
    // returned the count of the other two, so they read the completed states.
    __shared__ int last;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's state stores are complete
    __syncthreads();
    if (threadIdx.x == 0)
      last = __hip_atomic_fetch_add(cnt + b * gridDim.y + h, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             kAttnSplits - 1;
    __syncthreads();
    if (last) {
      const long long slot0 = slot - split;
      const float* po0 = part + slot0 * rows * D;
      const float* pml0 =
          part + static_cast<long long>(gridDim.x) * gridDim.y * kAttnSplits * rows * D + slot0 * rows * 2;
      for (int i = threadIdx.x; i < rows * D; i += blockDim.x) {
        const int r = i / D, c = i - r * D;
        out[(static_cast<long long>(b) * rows + r) * H + h * D + c] =
            from_f32<WT>(merge_splits(po0, pml0, rows, D, r, c, ld_agent));
      }
      if (threadIdx.x == 0)
        __hip_atomic_store(cnt + b * gridDim.y + h, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// out = the splits' states merged in split order, normalised; one workgroup
// per (sequence, head).  OT: fp32, or the cache type when the output feeds
// the output projection directly (rounded once at the store).
template <typename OT>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part, int rows, int H,
                                                         int D, OT* __restrict__ out) {
#pragma clang fp contract(off)
  const int b = blockIdx.x, h = blockIdx.y;
  const long long slot0 = (static_cast<long long>(b) * gridDim.y + h) * kAttnSplits;
  const float* po = part + slot0 * rows * D;
  const float* pml = part + static_cast<long long>(gridDim.x) * gridDim.y * kAttnSplits * rows * D + slot0 * rows * 2;
  for (int i = threadIdx.x; i < rows * D; i += 256) {
    const int r = i / D, c = i - r * D;
    out[(static_cast<long long>(b) * rows + r) * H + h * D + c] =
        from_f32<OT>(merge_splits(po, pml, rows, D, r, c, [](const float* p) { return *p; }));
  }
}

template <typename WT, int D, bool FUSE>
void launch_attn_d(const float* q, const WT* k, const WT* v, const int32_t* pos, int B, int rows, int max_len,
                   int H, int n_heads, float scale, float* part, int* cnt, WT* out, hipStream_t s) {
  const dim3 grid(B, n_heads, kAttnSplits);
  const dim3 block(kWave * kAttnWaves);
  if (rows <= 1)
    attn_decode_kernel<WT, D, 1, FUSE><<<grid, block, 0, s>>>(q, k, v, pos, rows, max_len, H, scale, part, cnt, out);
  else if (rows <= 4)
    attn_decode_kernel<WT, D, 4, FUSE><<<grid, block, 0, s>>>(q, k, v, pos, rows, max_len, H, scale, part, cnt, out);
  else if (rows <= 8)
    attn_decode_kernel<WT, D, 8, FUSE><<<grid, block, 0, s>>>(q, k, v, pos, rows, max_len, H, scale, part, cnt, out);
  else
    attn_decode_kernel<WT, D, 16, FUSE><<<grid, block, 0, s>>>(q, k, v, pos, rows, max_len, H, scale, part, cnt,
                                                               out);
}

template <typename WT, bool FUSE>
void launch_attn_t(const float* q, const void* kc, const void* vc, const int32_t* pos, int B, int rows,
                   int max_len, int H, int n_heads, float* part, int* cnt, void* out, hipStream_t s) {
  const int D = H / n_heads;
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  const WT* k = static_cast<const WT*>(kc);
  const WT* v = static_cast<const WT*>(vc);
  WT* o = static_cast<WT*>(out);
  switch (D) {
    case 64: launch_attn_d<WT, 64, FUSE>(q, k, v, pos, B, rows, max_len, H, n_heads, scale, part, cnt, o, s); break;
    case 128: launch_attn_d<WT, 128, FUSE>(q, k, v, pos, B, rows, max_len, H, n_heads, scale, part, cnt, o, s); break;
    case 256: launch_attn_d<WT, 256, FUSE>(q, k, v, pos, B, rows, max_len, H, n_heads, scale, part, cnt, o, s); break;
    default: break;  // validated
  }
}

}  // namespace

size_t attn_ws_bytes(int B, int rows, int H, int n_heads) {
  return static_cast<size_t>(B) * kAttnSplits * rows * (H + 2 * n_heads) * sizeof(float);
}

void launch_attn_decode(const float* q, const void* k_cache, const void* v_cache, const int32_t* pos,
                        int B, int rows, int max_len, int H, int n_heads, int dt, void* out, bool out_dt,
                        float* part, hipStream_t s, int* fuse_cnt) {
  if (fuse_cnt != nullptr && out_dt) {
    // the last split of each (sequence, head) merges: no second launch
    if (dt == MOEV_BF16)
      launch_attn_t<u16, true>(q, k_cache, v_cache, pos, B, rows, max_len, H, n_heads, part, fuse_cnt, out, s);
    else
      launch_attn_t<float, true>(q, k_cache, v_cache, pos, B, rows, max_len, H, n_heads, part, fuse_cnt, out, s);
    return;
  }
  if (dt == MOEV_BF16)
    launch_attn_t<u16, false>(q, k_cache, v_cache, pos, B, rows, max_len, H, n_heads, part, nullptr, nullptr, s);
  else
    launch_attn_t<float, false>(q, k_cache, v_cache, pos, B, rows, max_len, H, n_heads, part, nullptr, nullptr, s);
  const dim3 grid(B, n_heads);
  const int D = H / n_heads;
  if (out_dt && dt == MOEV_BF16)
    attn_merge_kernel<u16><<<grid, 256, 0, s>>>(part, rows, H, D, static_cast<u16*>(out));
  else
    attn_merge_kernel<float><<<grid, 256, 0, s>>>(part, rows, H, D, static_cast<float*>(out));
}

}  // namespace moev

extern "C" size_t moev_attn_decode_workspace_size(int B, int rows, int H, int n_heads) {
  if (B < 0 || rows < 1 || n_heads < 1 || H < 1) return 0;
  return moev::attn_ws_bytes(B, rows, H, n_heads);
}

extern "C" moev_status moev_attn_decode(const float* q, const void* k_cache, const void* v_cache,
                                        const int32_t* pos, int B, int rows, int max_len, int H,
                                        int n_heads, int dt, float* out, void* ws, size_t ws_bytes,
                                        void* stream) {
  using namespace moev;
  clear_error();
  MOEV_CHECK(check_dtype(dt), MOEV_ERR_UNSUPPORTED);
  MOEV_REQUIRE(B >= 0, MOEV_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
  MOEV_REQUIRE(rows >= 1 && rows <= kAttnMaxRows, MOEV_ERR_UNSUPPORTED, "rows=%d must be in [1, %d]", rows,
               kAttnMaxRows);
  MOEV_REQUIRE(n_heads >= 1 && H >= 1 && H % n_heads == 0, MOEV_ERR_UNSUPPORTED,
               "H=%d must be a positive multiple of n_heads=%d", H, n_heads);
  const int D = H / n_heads;
  MOEV_REQUIRE(D == 64 || D == 128 || D == 256, MOEV_ERR_UNSUPPORTED,
               "head width %d must be 64, 128 or 256", D);
  MOEV_REQUIRE(max_len >= rows, MOEV_ERR_INVALID_ARG, "max_len=%d must be >= rows=%d", max_len, rows);
  if (B == 0) return MOEV_OK;
  MOEV_CHECK(need_ptr(q, "q") && need_ptr(k_cache, "k_cache") && need_ptr(v_cache, "v_cache") &&
                 need_ptr(pos, "pos", 4) && need_ptr(out, "out"),
             MOEV_ERR_INVALID_ARG);
  const size_t need = attn_ws_bytes(B, rows, H, n_heads);
  MOEV_REQUIRE(ws != nullptr && aligned16(ws), MOEV_ERR_WORKSPACE, "workspace must be non-NULL and 16-byte aligned");
  MOEV_REQUIRE(ws_bytes >= need, MOEV_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  launch_attn_decode(q, k_cache, v_cache, pos, B, rows, max_len, H, n_heads, dt, out, false,
                     static_cast<float*>(ws), as_stream(stream));
  return launch_status("moev_attn_decode");
}
