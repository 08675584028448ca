// Lightning Indexer scoring and per-query top-k selection for gfx950.
//
// Source: DeepSeek-V4 model page (Transformers docs), "Hybrid attention (§2.3)", CSA item
// (the indexer scores each query against the pooled entries and keeps index_topk of them,
// eqs. 13-17) and "Attention mask layout", CSA paragraph (-1 sentinel for empty slots;
// entry w is visible to query t iff w < (t+1)//m).
//
// Score (reading R8): score[t,w] = sum_h w_idx[t,h] * max(0, q_idx[t,h,:] . k_pool[w,:]).
// Selection (reading R9): the min(k, V) largest scores, ties to the lower entry index, -0
// ranked as +0, emitted in ascending entry order followed by -1.
#include "common.h"
#include "launch.h"

namespace dsv4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

namespace {

constexpr int IX_NI = 64;     // indexer heads covered by the MFMA path
constexpr int IX_CI = 128;    // indexer head dim covered by the MFMA path
constexpr int IX_TILE = 128;  // pool entries per LDS tile (4 sub-tiles of 32)
constexpr int IX_PITCH = IX_CI * 2 + 16;  // LDS bytes per entry row (16 B pad spreads banks)

__device__ __forceinline__ int visible_entries(const int* q_pos0, const int* n_pool, int b, int t,
                                               int m, int N_cap) {
  long long v = (static_cast<long long>(q_pos0[b]) + t + 1) / m;
  v = min(v, static_cast<long long>(n_pool[b]));
  v = min(v, static_cast<long long>(N_cap));
  return static_cast<int>(max(v, 0LL));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

}  // namespace

// ---------------------------------------------------------------------------
// MFMA scoring (bf16, 64 heads x 128 dims).  S = Q . K^T per query on
// v_mfma_f32_32x32x16_bf16: A = Q (32 heads x 16 dims, registers), B = K^T (16 dims x 32
// entries, LDS).  The C tile holds 16 heads of one entry per lane, so the ReLU-weighted head
// sum is 16 local FMAs and one cross-half shuffle.
//
// SPLIT = false (prefill): a block owns 4*QPW consecutive queries (QPW per wave); all waves
//   walk the same 128-entry tiles, so each LDS tile is reused by every query of the block.
// SPLIT = true (decode, one query per block): the block owns a chunk of tiles; wave w scores
//   sub-tile w of every tile.
// ---------------------------------------------------------------------------
template <int QPW, bool SPLIT>
__global__ void __launch_bounds__(256, 1) index_score_mfma(
    const bf16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const bf16_t* __restrict__ k_pool, const int* __restrict__ q_pos0,
    const int* __restrict__ n_pool, float* __restrict__ scores, int T, int N_cap, int m,
    int tiles_per_chunk) {
  __shared__ __attribute__((aligned(16))) unsigned char ktile[IX_TILE * IX_PITCH];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int b = blockIdx.z;
  constexpr int QB = SPLIT ? 1 : 4 * QPW;
  // heaviest (latest) query blocks first
  const int t0 = SPLIT ? blockIdx.x : (gridDim.x - 1 - blockIdx.x) * QB;

  int tq[QPW], V[QPW];
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi) {
    tq[qi] = SPLIT ? t0 : t0 + wave * QPW + qi;
    V[qi] = tq[qi] < T ? visible_entries(q_pos0, n_pool, b, tq[qi], m, N_cap) : 0;
  }
  const int t_last = min(t0 + QB - 1, T - 1);
  const int Vmax = visible_entries(q_pos0, n_pool, b, t_last, m, N_cap);
  const int n_tiles = (Vmax + IX_TILE - 1) / IX_TILE;
  int tile_begin = 0, tile_end = n_tiles;
  if (SPLIT) {
    tile_begin = blockIdx.y * tiles_per_chunk;
    tile_end = min(n_tiles, tile_begin + tiles_per_chunk);
  }
  if (tile_begin >= tile_end) return;  // block-uniform

  // Q fragments and head weights of this wave's queries
  bf16x8_t qa[QPW][2][IX_CI / 16];
  float wv[QPW][2][16];
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi) {
    const int t = min(tq[qi], T - 1);
    const size_t qrow = static_cast<size_t>(b) * T + t;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const bf16_t* qp = q_idx + (qrow * IX_NI + hb * 32 + l32) * IX_CI + half * 8;
#pragma unroll
      for (int ks = 0; ks < IX_CI / 16; ++ks)
        qa[qi][hb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + ks * 16));
      const float* wp = w_idx + qrow * IX_NI + hb * 32 + half * 4;
#pragma unroll
      for (int e = 0; e < 16; ++e) wv[qi][hb][e] = wp[(e >> 2) * 8 + (e & 3)];
    }
  }

  const bf16_t* kbase = k_pool + static_cast<size_t>(b) * N_cap * IX_CI;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int n0 = tile * IX_TILE;
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int pass = 0; pass < IX_TILE * IX_CI * 2 / (256 * 16); ++pass) {
      const int row = pass * 16 + (threadIdx.x >> 4);
      const int ch = threadIdx.x & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n0 + row < N_cap)
        v = *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(n0 + row) * IX_CI + ch * 8);
      *reinterpret_cast<uint4*>(ktile + row * IX_PITCH + ch * 16) = v;
    }
    __syncthreads();

#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      if (SPLIT && sub != wave) continue;
      f32x16_t acc[QPW][2];
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[qi][hb][e] = 0.f;
      const unsigned char* brow = ktile + (sub * 32 + l32) * IX_PITCH + half * 16;
#pragma unroll
      for (int ks = 0; ks < IX_CI / 16; ++ks) {
        const bf16x8_t bk = *reinterpret_cast<const bf16x8_t*>(brow + ks * 32);
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
            acc[qi][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[qi][hb][ks], bk, acc[qi][hb], 0, 0, 0);
      }
      const int n = n0 + sub * 32 + l32;
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        float part = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 16; ++e) part += wv[qi][hb][e] * fmaxf(acc[qi][hb][e], 0.f);
        part += __shfl_xor(part, 32);
        if (half == 0 && n < V[qi])
          scores[(static_cast<size_t>(b) * T + tq[qi]) * N_cap + n] = part;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Generic scoring (any nI, cI, fp32 or bf16): one block per query, one thread per entry.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) index_score_generic(
    const T* __restrict__ q_idx, const float* __restrict__ w_idx, const T* __restrict__ k_pool,
    const int* __restrict__ q_pos0, const int* __restrict__ n_pool, float* __restrict__ scores,
    int Tq, int nI, int cI, int N_cap, int m) {
  extern __shared__ float sq[];  // q row [nI*cI], then w [nI]
  const int qrow = blockIdx.x;
  const int b = qrow / Tq, t = qrow % Tq;
  const int V = visible_entries(q_pos0, n_pool, b, t, m, N_cap);
  const T* qp = q_idx + static_cast<size_t>(qrow) * nI * cI;
  for (int i = threadIdx.x; i < nI * cI; i += blockDim.x) sq[i] = load1<T>(qp + i);
  for (int i = threadIdx.x; i < nI; i += blockDim.x) sq[nI * cI + i] = w_idx[static_cast<size_t>(qrow) * nI + i];
  __syncthreads();
  for (int n = threadIdx.x; n < V; n += blockDim.x) {
    const T* kr = k_pool + (static_cast<size_t>(b) * N_cap + n) * cI;
    float tot = 0.f;
    for (int h = 0; h < nI; ++h) {
      float dot = 0.f;
      for (int c = 0; c < cI; ++c) dot += sq[h * cI + c] * load1<T>(kr + c);
      tot += sq[nI * cI + h] * fmaxf(dot, 0.f);
    }
    scores[static_cast<size_t>(qrow) * N_cap + n] = tot;
  }
}

bool index_scores_fast(int nI, int cI, int dtype) { return dtype == 1 && nI == IX_NI && cI == IX_CI; }

hipError_t launch_index_scores(const void* q_idx, const float* w_idx, const void* k_pool,
                               const int* q_pos0, const int* n_pool, float* scores, int B, int T,
                               int nI, int cI, int N_cap, int m, int dtype, hipStream_t st) {
  if (T == 0 || B == 0) return hipSuccess;
  if (index_scores_fast(nI, cI, dtype)) {
    const bf16_t* qp = static_cast<const bf16_t*>(q_idx);
    const bf16_t* kp = static_cast<const bf16_t*>(k_pool);
    if (T >= 8) {
      constexpr int QPW = 2;
      dim3 grid(div_up(T, 4 * QPW), 1, B);
      hipLaunchKernelGGL((index_score_mfma<QPW, false>), grid, dim3(256), 0, st, qp, w_idx, kp,
                         q_pos0, n_pool, scores, T, N_cap, m, 0);
    } else {
      // one query per block, entry tiles split over blocks (decode-sized T)
      const int tiles = (N_cap + IX_TILE - 1) / IX_TILE;
      const int tpc = 8;  // 1024 entries per block
      dim3 grid(T, div_up(tiles, tpc), B);
      hipLaunchKernelGGL((index_score_mfma<1, true>), grid, dim3(256), 0, st, qp, w_idx, kp,
                         q_pos0, n_pool, scores, T, N_cap, m, tpc);
    }
    return hipGetLastError();
  }
  const size_t shmem = static_cast<size_t>(nI * cI + nI) * sizeof(float);
  if (dtype == 1)
    hipLaunchKernelGGL((index_score_generic<bf16_t>), dim3(B * T), dim3(256), shmem, st,
                       static_cast<const bf16_t*>(q_idx), w_idx, static_cast<const bf16_t*>(k_pool),
                       q_pos0, n_pool, scores, T, nI, cI, N_cap, m);
  else
    hipLaunchKernelGGL((index_score_generic<float>), dim3(B * T), dim3(256), shmem, st,
                       static_cast<const float*>(q_idx), w_idx, static_cast<const float*>(k_pool),
                       q_pos0, n_pool, scores, T, nI, cI, N_cap, m);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k: radix select on order-preserving uint32 keys (4 passes of 8 bits, per-wave LDS
// histograms, block suffix scan to find each digit), then an index-ordered compaction that
// takes every key above the threshold and the lowest-index keys equal to it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NT>
__global__ void __launch_bounds__(NT) topk_kernel(const float* __restrict__ scores,
                                                  const int* __restrict__ q_pos0,
                                                  const int* __restrict__ n_pool,
                                                  int* __restrict__ topk_idx,
                                                  float* __restrict__ topk_score, int T, int N_cap,
                                                  int m, int k) {
  constexpr int NW = NT / 64;
  static_assert(NT >= 256, "one thread per histogram bin");
  __shared__ uint32_t hist[NW][256];
  __shared__ int scan_w[NW];
  __shared__ int wave_tot[NW];
  __shared__ int sh_digit, sh_above;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qrow = blockIdx.x;
  const int b = qrow / T, t = qrow % T;
  const int V = visible_entries(q_pos0, n_pool, b, t, m, N_cap);
  const float* s = scores + static_cast<size_t>(qrow) * N_cap;
  const int kk = min(k, V);
  const bool take_all = (kk == V);
  uint32_t prefix = 0, mask = 0;
  int remaining = kk;

  if (!take_all) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < NW * 256; i += NT) (&hist[0][0])[i] = 0;
      __syncthreads();
      for (int i = tid; i < V; i += NT) {
        const uint32_t key = score_key(s[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // suffix sums over the 256 bins: thread j < 256 holds bin d = 255 - j
      int cnt = 0, incl = 0;
      if (tid < 256) {
        const int d = 255 - tid;
#pragma unroll
        for (int w = 0; w < NW; ++w) cnt += static_cast<int>(hist[w][d]);
        incl = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int v = __shfl_up(incl, off);
          if (lane >= off) incl += v;
        }
        if (lane == 63) scan_w[wave] = incl;
      }
      __syncthreads();
      if (tid < 256) {
        for (int w = 0; w < wave; ++w) incl += scan_w[w];
        const int above = incl - cnt;  // keys with a larger digit
        if (above < remaining && remaining <= incl) { sh_digit = 255 - tid; sh_above = above; }
      }
      __syncthreads();
      const uint32_t d = static_cast<uint32_t>(sh_digit);
      remaining -= sh_above;
      prefix |= d << shift;
      mask |= 255u << shift;
      __syncthreads();
    }
  }

  // index-ordered compaction
  int* out_i = topk_idx + static_cast<size_t>(qrow) * k;
  float* out_s = topk_score ? topk_score + static_cast<size_t>(qrow) * k : nullptr;
  int out_base = 0, eq_base = 0;
  for (int base = 0; base < V; base += NT) {
    const int i = base + tid;
    const bool valid = i < V;
    const float sv = valid ? s[i] : 0.f;
    bool sel;
    if (take_all) {
      sel = valid;
    } else {
      const uint32_t key = score_key(sv);
      const bool gt = valid && key > prefix;
      const bool eq = valid && key == prefix;
      int eq_tot;
      const int eq_rank = eq_base + block_excl_count<NT>(eq, &eq_tot, wave_tot);
      eq_base += eq_tot;
      sel = gt || (eq && eq_rank < remaining);
    }
    int sel_tot;
    const int pos = out_base + block_excl_count<NT>(sel, &sel_tot, wave_tot);
    out_base += sel_tot;
    if (sel && pos < k) {
      out_i[pos] = i;
      if (out_s) out_s[pos] = sv;
    }
  }
  for (int p = kk + tid; p < k; p += NT) {
    out_i[p] = -1;
    if (out_s) out_s[p] = 0.f;
  }
}

hipError_t launch_topk(const float* scores, const int* q_pos0, const int* n_pool, int* topk_idx,
                       float* topk_score, int B, int T, int N_cap, int m, int k, hipStream_t st) {
  if (B == 0 || T == 0) return hipSuccess;
  if (N_cap > 8192)
    hipLaunchKernelGGL((topk_kernel<1024>), dim3(B * T), dim3(1024), 0, st, scores, q_pos0, n_pool,
                       topk_idx, topk_score, T, N_cap, m, k);
  else
    hipLaunchKernelGGL((topk_kernel<256>), dim3(B * T), dim3(256), 0, st, scores, q_pos0, n_pool,
                       topk_idx, topk_score, T, N_cap, m, k);
  return hipGetLastError();
}

}  // namespace dsv4
