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

__device__ __forceinline__ int visible_entries(const int* q_pos0, const int* n_pool, int b, int t,
                                               int m, int N_cap) {
  long long v = (static_cast<long long>(q_pos0[b]) + t + 1) / m;
  v = min(v, static_cast<long long>(n_pool[b]));
  v = min(v, static_cast<long long>(N_cap));
  return static_cast<int>(max(v, 0LL));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

constexpr int IX_ROW = IX_CI * 2;  // bytes per indexer key row

// Raw buffer descriptor over [base, base + bytes): reads past the end return zeros.  The
// arguments are made wave-uniform explicitly, so the descriptor lives in SGPRs (a descriptor
// the compiler cannot prove uniform is applied lane group by lane group in a loop).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ rsrc_t make_rs(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32));
  void* p = reinterpret_cast<void*>((static_cast<unsigned long long>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, static_cast<short>(0),
                                           static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)),
                                           0x00020000);
}

// Sum of a value across the two 32-lane halves of the wave.
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

// ---------------------------------------------------------------------------
// MFMA scoring (bf16, 64 heads x 128 dims).  S = Q . K^T per query on
// v_mfma_f32_32x32x16_bf16: A = Q (32 heads x 16 dims, registers), B = K^T (16 dims x 32
// entries).  The C tile holds 16 heads of one entry per lane, so the ReLU-weighted head sum
// is 16 local FMAs and one cross-half shuffle.
//
// Prefill (index_score_mfma): a block owns NWV = 4 consecutive queries, one per wave (one
// per SIMD); all its waves walk the same 128-entry LDS tiles, so each tile is reused by every
// query of the block.  Two blocks share a CU (two waves per SIMD, so one wave's ReLU-weighted
// head sums overlap the other's MFMAs) and wait at their tile barriers independently, which
// measured ~6 % faster than one block of 8 waves sharing one barrier.
// ---------------------------------------------------------------------------
template <int NWV>
__global__ void __launch_bounds__(256, 2) index_score_mfma(
    const bf16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const bf16_t* __restrict__ k_pool, const int* __restrict__ q_pos0,
    const int* __restrict__ n_pool, float* __restrict__ scores, int T, int N_cap, int m) {
  // two tile slots: tile s+1 streams into one (LDS-DMA) while tile s is read from the other
  __shared__ __attribute__((aligned(16))) unsigned char ktile[2][IX_TILE * IX_ROW];
  static_assert(NWV == 4, "launch bounds are written for 4 waves");
  constexpr int LPW = 8;  // LDS-DMA instructions (1 KB each) per wave per tile
  static_assert(LPW * NWV * 1024 == IX_TILE * IX_ROW, "waves x instructions cover a tile");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int b = blockIdx.z;
  // heaviest (latest) query blocks first; wave w scores query t0 + w
  const int t0 = (gridDim.x - 1 - blockIdx.x) * NWV;
  const int tq = t0 + wave;
  const int V = tq < T ? visible_entries(q_pos0, n_pool, b, tq, m, N_cap) : 0;
  const int t_last = min(t0 + NWV - 1, T - 1);
  const int Vmax = visible_entries(q_pos0, n_pool, b, t_last, m, N_cap);
  const int n_tiles = (Vmax + IX_TILE - 1) / IX_TILE;
  if (n_tiles == 0) return;  // block-uniform

  // Tile loads: LDS chunk p (16 bytes) of a slot holds chunk c = (p & 15) ^ (row & 15) of entry
  // row = p >> 4, so the B-operand reads (32 rows, one chunk column) hit 16 distinct bank
  // groups.  Wave w fills chunks 64*LPW*w .. (LPW instructions of 64 lanes).  Rows past N_cap
  // lie beyond the buffer descriptor and read as zeros.
  const rsrc_t krs = make_rs(k_pool + static_cast<size_t>(b) * N_cap * IX_CI,
                             static_cast<unsigned>(N_cap) * IX_ROW);
  unsigned soff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int p = (wave * LPW + j) * 64 + lane;
    const int row = p >> 4;
    soff[j] = static_cast<unsigned>(row * IX_ROW + (((p & 15) ^ (row & 15)) << 4));
  }
  auto issue = [&](int tile, int slot) {
    const unsigned base = static_cast<unsigned>(tile) * (IX_TILE * IX_ROW);
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krs, (lds_void*)(&ktile[slot][(wave * LPW + j) * 1024]), 16, soff[j] + base, 0, 0, 0);
  };
  issue(0, 0);

  // Q fragments and head weights of this wave's query
  bf16x8_t qa[2][IX_CI / 16];
  float wv[2][16];
  {
    const size_t qrow = static_cast<size_t>(b) * T + min(tq, T - 1);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const bf16_t* qp = q_idx + (qrow * IX_NI + hb * 32 + l32) * IX_CI + half * 8;
#pragma unroll
      for (int ks = 0; ks < IX_CI / 16; ++ks)
        qa[hb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + ks * 16));
      const float* wp = w_idx + qrow * IX_NI + hb * 32 + half * 4;
#pragma unroll
      for (int e = 0; e < 16; ++e) wv[hb][e] = wp[(e >> 2) * 8 + (e & 3)];
    }
  }
  // Score stores go through a descriptor over this query's row: lanes with nothing to store
  // get an offset past its end, so every sub-tile issues exactly one store instruction and
  // the tile loop can wait for its LDS-DMA loads without waiting for the stores behind them.
  const rsrc_t srs = make_rs(scores + (static_cast<size_t>(b) * T + min(tq, T - 1)) * N_cap,
                             static_cast<unsigned>(N_cap) * 4u);
  const int rsw = l32 & 15;  // B-operand chunk swizzle of this lane's row

  // Software pipeline over 32-entry sub-tiles: the MFMAs of sub-tile j and the ReLU-weighted
  // head sum of sub-tile j-1 (two accumulator sets) are independent, so the compiler
  // interleaves them; the first four B fragments of sub-tile j+1 are read from LDS during
  // sub-tile j's MFMAs.  (Fixed scheduling groups of 2 MFMAs : 9 VALU with all 8 fragment
  // reads first were ~4 % slower: each sub-tile then began by waiting for its reads.)
  f32x16_t accA[2], accB[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int e = 0; e < 16; ++e) accB[hb][e] = 0.f;
  int n_pend = -1;  // entry of this lane's pending score (none yet)
  const f32x16_t zero = {};

  bf16x8_t bpre[4];  // the first four B fragments of the next sub-tile of this tile
  auto frag = [&](const unsigned char* kt, int sub, int ks) {
    return *reinterpret_cast<const bf16x8_t*>(kt + (sub * 32 + l32) * IX_ROW + (((2 * ks + half) ^ rsw) << 4));
  };
  auto scores_of = [&](f32x16_t (&acc)[2], const unsigned char* kt, int sub) {
    bf16x8_t bk[IX_CI / 16];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bk[ks] = sub == 0 ? frag(kt, sub, ks) : bpre[ks];
#pragma unroll
    for (int ks = 4; ks < IX_CI / 16; ++ks) bk[ks] = frag(kt, sub, ks);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
      acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[hb][0], bk[0], zero, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < IX_CI / 16; ++ks) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[hb][ks], bk[ks], acc[hb], 0, 0, 0);
      if (ks == 3 && sub < 3) {
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) bpre[k2] = frag(kt, sub + 1, k2);
      }
    }
  };
  // ReLU as an integer max: non-negative floats are non-negative integers, and -0 -> +0
  auto head_sum = [&](const f32x16_t (&acc)[2], int n) {
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      p0 += wv[0][e] * __int_as_float(max(__float_as_int(acc[0][e]), 0));
      p1 += wv[1][e] * __int_as_float(max(__float_as_int(acc[1][e]), 0));
      p2 += wv[0][e + 1] * __int_as_float(max(__float_as_int(acc[0][e + 1]), 0));
      p3 += wv[1][e + 1] * __int_as_float(max(__float_as_int(acc[1][e + 1]), 0));
    }
    const float part = xhalf_sum((p0 + p1) + (p2 + p3));
    const bool ok = half == 0 && n >= 0 && n < V;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part), srs,
                                          ok ? static_cast<unsigned>(n) * 4u : 0xFFFFFFF0u, 0, 0);
  };

  bool stored = false;  // the previous tile issued its 4 score stores after its loads
  for (int tile = 0; tile < n_tiles; ++tile) {
    // This wave's part of tile `tile` has landed: vector memory operations complete in issue
    // order, and only the previous tile's 4 score stores were issued after those loads.  After
    // the barrier every part has, and every wave is past tile-1, whose slot is reused.
    if (stored)
      __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tile + 1 < n_tiles) issue(tile + 1, (tile + 1) & 1);
    const unsigned char* kt = ktile[tile & 1];
    const int n0 = tile * IX_TILE;
    stored = n0 < V;
    if (!stored) continue;  // wave-uniform: this query sees none of the tile (only at the end)

    scores_of(accA, kt, 0);
    head_sum(accB, n_pend);
    scores_of(accB, kt, 1);
    head_sum(accA, n0 + l32);
    scores_of(accA, kt, 2);
    head_sum(accB, n0 + 32 + l32);
    scores_of(accB, kt, 3);
    head_sum(accA, n0 + 64 + l32);
    n_pend = n0 + 96 + l32;
  }
  head_sum(accB, n_pend);
}

// ---------------------------------------------------------------------------
// Decode-sized T (index_score_stream): the scan is bound by reading the indexer keys once
// (64 flops per byte), so every wave streams its own EPW consecutive entries of one query
// straight from HBM into B-operand registers, one 32-entry sub-tile ahead of the MFMAs.  No
// LDS, no barriers: waves are independent and many are resident, which keeps enough key
// bytes in flight to cover HBM latency.  Lane (l32, half) loads 16 bytes of entry row l32 per
// 16-dim step; the 8 steps of a sub-tile together read whole 256-byte rows.
// ---------------------------------------------------------------------------
// Scores of entries [e0, e1) of query (b, t) (e0 < e1 <= its visible count), streamed by one
// wave: lane (l32, half) loads 16 bytes of entry row l32 per 16-dim step, the 8 steps of a
// sub-tile together read whole 256-byte rows; three register sets rotate, so sub-tiles n0 + 32
// and n0 + 64 are in flight while n0 is scored.
__device__ __forceinline__ void stream_scores(const bf16_t* __restrict__ q_idx,
                                              const float* __restrict__ w_idx,
                                              const bf16_t* __restrict__ k_pool,
                                              float* __restrict__ scores, int b, int t, int T,
                                              int N_cap, int e0, int e1) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const size_t qrow = static_cast<size_t>(b) * T + t;

  bf16x8_t qa[2][IX_CI / 16];
  float wv[2][16];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const bf16_t* qp = q_idx + (qrow * IX_NI + hb * 32 + l32) * IX_CI + half * 8;
#pragma unroll
    for (int ks = 0; ks < IX_CI / 16; ++ks)
      qa[hb][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + ks * 16));
    const float* wp = w_idx + qrow * IX_NI + hb * 32 + half * 4;
#pragma unroll
    for (int e = 0; e < 16; ++e) wv[hb][e] = wp[(e >> 2) * 8 + (e & 3)];
  }

  // rows past e1 are clamped to e1 - 1 (a visible row): loads stay in bounds, results unused
  const bf16_t* kb = k_pool + static_cast<size_t>(b) * N_cap * IX_CI + half * 8;
  float* srow = scores + qrow * N_cap;
  auto load = [&](uint4 (&dst)[IX_CI / 16], int n) {
    const bf16_t* kr = kb + static_cast<size_t>(min(n + l32, e1 - 1)) * IX_CI;
#pragma unroll
    for (int ks = 0; ks < IX_CI / 16; ++ks) dst[ks] = *reinterpret_cast<const uint4*>(kr + ks * 16);
  };
  auto score = [&](const uint4 (&src)[IX_CI / 16], int n0) {
    f32x16_t acc[2];
    const f32x16_t zero = {};
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
      acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[hb][0], as_bf16x8(src[0]), zero, 0, 0, 0);
#pragma unroll
    for (int ks = 1; ks < IX_CI / 16; ++ks)
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[hb][ks], as_bf16x8(src[ks]), acc[hb], 0, 0, 0);
    // ReLU as an integer max: non-negative floats are non-negative integers, and -0 -> +0
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p0 += wv[0][e] * __int_as_float(max(__float_as_int(acc[0][e]), 0));
      p1 += wv[1][e] * __int_as_float(max(__float_as_int(acc[1][e]), 0));
    }
    const float part = xhalf_sum(p0 + p1);
    const int n = n0 + l32;
    if (half == 0 && n < e1) srow[n] = part;
  };
  uint4 b0[IX_CI / 16], b1[IX_CI / 16], b2[IX_CI / 16];
  // The Q and head-weight loads stay ahead of the key loads (the scheduler moved some after
  // them), so that the wait below leaves only the 16 key loads in flight.  Otherwise the
  // Q fragments and head weights count as loads still in flight inside the loop, and each
  // use waited for every key load issued since: every sub-tile drained the queue.
  __builtin_amdgcn_sched_barrier(0);
  load(b0, e0);
  load(b1, e0 + 32);  // rows clamped: in bounds even past e1
  __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): Q fragments and head weights landed
  // Every load and score of the loop is unconditional: past e1 the loads read the clamped
  // last row (in bounds, cached) and the stores are masked.  With conditional loads the
  // compiler's waits, merged over the paths that skip them, treated the sub-tile about to be
  // scored as the latest load and drained the two issued after it.
  for (int n0 = e0; n0 < e1; n0 += 96) {  // wave-uniform bounds throughout
    load(b2, n0 + 64);
    score(b0, n0);
    load(b0, n0 + 96);
    score(b1, n0 + 32);
    load(b1, n0 + 128);
    score(b2, n0 + 64);
  }
}

// Decode-sized T, many rows (index_score_stream): the scan is bound by reading the indexer keys
// once (64 flops per byte), so every wave streams its own EPW consecutive entries of one query
// straight from HBM into B-operand registers.  No LDS, no barriers.
template <int EPW>
__global__ void __launch_bounds__(256) index_score_stream(
    const bf16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const bf16_t* __restrict__ k_pool, const int* __restrict__ q_pos0,
    const int* __restrict__ n_pool, float* __restrict__ scores, int T, int N_cap, int m) {
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.y, b = blockIdx.z;
  const int V = visible_entries(q_pos0, n_pool, b, t, m, N_cap);
  const int e0 = (blockIdx.x * 4 + wave) * EPW;
  if (e0 >= V) return;  // wave-uniform
  stream_scores(q_idx, w_idx, k_pool, scores, b, t, T, N_cap, e0, min(V, e0 + EPW));
}

// Decode-sized T, up to kScanMaxRows rows (index_score_scan): a persistent grid whose waves
// each take an equal share of all rows' 32-entry sub-tiles, as one contiguous range (part of a
// row, or the end of one row and the start of the next).  A fixed number of entries per wave
// would leave the device partly idle in the last round of waves; here every wave ends within
// one sub-tile of the others.  Each block first forms the rows' sub-tile counts and their
// prefix in LDS.
constexpr int kScanMaxRows = 2048;
__global__ void __launch_bounds__(256) index_score_scan(
    const bf16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const bf16_t* __restrict__ k_pool, const int* __restrict__ q_pos0,
    const int* __restrict__ n_pool, float* __restrict__ scores, int T, int N_cap, int m, int rows) {
  constexpr int RPT = kScanMaxRows / 256;
  __shared__ int pre[kScanMaxRows + 1];  // sub-tiles of the rows before row r
  __shared__ int wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // thread tid owns rows rpt*tid .. rpt*tid + rpt - 1 (one row each up to 256 rows); every
  // position load is issued before any count is formed (one memory round trip, not one per row)
  const int rpt = (rows + 255) / 256;
  int qp[RPT], np[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int b = min(tid * rpt + j, rows - 1) / T;
    qp[j] = q_pos0[b];
    np[j] = n_pool[b];
  }
  int cnt[RPT];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int r = tid * rpt + j;
    long long v = (static_cast<long long>(qp[j]) + r % T + 1) / m;  // visible_entries, inlined
    v = min(min(v, static_cast<long long>(np[j])), static_cast<long long>(N_cap));
    cnt[j] = (j < rpt && r < rows) ? (static_cast<int>(max(v, 0LL)) + 31) / 32 : 0;
    mine += cnt[j];
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int run = incl - mine, total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    run += w < wave ? wtot[w] : 0;
    total += wtot[w];
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int r = tid * rpt + j;
    if (j < rpt && r < rows) pre[r] = run;
    run += cnt[j];
  }
  if (tid == 0) pre[rows] = total;
  __syncthreads();

  const long long W = static_cast<long long>(gridDim.x) * 4;
  const long long wid = static_cast<long long>(blockIdx.x) * 4 + wave;
  int s = static_cast<int>(total * wid / W);
  const int s1 = static_cast<int>(total * (wid + 1) / W);
  if (s >= s1) return;  // wave-uniform
  // the row holding sub-tile s: the last r with pre[r] <= s
  int r = 0, hi = rows - 1;
  while (r < hi) {
    const int mid = (r + hi + 1) >> 1;
    if (pre[mid] <= s) r = mid;
    else hi = mid - 1;
  }
  while (s < s1) {
    while (pre[r + 1] <= s) ++r;  // rows without entries
    const int end = min(s1, pre[r + 1]);
    const int b = r / T, t = r % T;
    const int V = visible_entries(q_pos0, n_pool, b, t, m, N_cap);
    stream_scores(q_idx, w_idx, k_pool, scores, b, t, T, N_cap, (s - pre[r]) * 32,
                  min(V, (end - pre[r]) * 32));
    s = end;
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
      constexpr int NWV = 4;  // queries per block, one per wave
      dim3 grid(div_up(T, NWV), 1, B);
      hipLaunchKernelGGL((index_score_mfma<NWV>), grid, dim3(NWV * 64), 0, st, qp, w_idx, kp,
                         q_pos0, n_pool, scores, T, N_cap, m);
    } else if (B * T <= kScanMaxRows) {
      // decode-sized T: a persistent grid (two blocks of four waves per CU) over every row
      static int n_cu = 0;
      if (n_cu == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
          n_cu = n;
        else
          return hipErrorInvalidDevice;
      }
      hipLaunchKernelGGL(index_score_scan, dim3(2 * n_cu), dim3(256), 0, st, qp, w_idx, kp, q_pos0,
                         n_pool, scores, T, N_cap, m, B * T);
    } else {
      // decode-sized T, many rows: one query per block row, 4 waves x EPW entries per block
      constexpr int EPW = 256;
      dim3 grid(div_up(N_cap, 4 * EPW), T, B);
      hipLaunchKernelGGL((index_score_stream<EPW>), grid, dim3(256), 0, st, qp, w_idx, kp, q_pos0,
                         n_pool, scores, T, N_cap, m);
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
// Top-k of one query row (one block per row).
//
// Keys: order-preserving uint32 images of the fp32 scores (-0 ranked as +0).  Thread tid
// owns indices j*NT + tid; the first KPT of them stay in registers, later ones are re-read
// (coalesced) from the score row on every pass.
//
// Threshold: radix select, most significant digit first.  The first digit (4 bits) is
// counted by every key: lane l of every wave counts into column l of a [16 digits][64
// lanes] LDS histogram, so the lanes of one atomic never collide whatever the score
// distribution, and wave d sums digit d's column with DPP moves.  The digits of 11, 11 and
// 6 bits after it are counted only by the keys that carry the digits chosen so far, in a
// 2048-bin histogram (a key outside them adds to a lane-private spare bin); a block scan of
// the threads' bin sums (thread t holds 2048/NT bins, the highest first) finds the wave, a
// wave scan the thread and a walk of its bins the digit.  A pass stops the search once the
// chosen bin holds exactly the keys still needed: on continuous scores after three passes,
// against five to seven of 4-bit digits.  Two histograms alternate, so one is cleared while
// the other is read; two barriers per pass.
//
// Output: index-ordered compaction through LDS bitmaps, segment by segment (32768 indices):
// one bit per key above the threshold and one per key equal to it (both from wave ballots;
// a wave collects the two words of its register stride j in lanes 2j, 2j + 1 and writes
// them with one LDS store per lane),
// a block scan of the equal-key popcounts keeps the lowest-index equal keys that are needed
// (ties to the lower entry index), and a block scan of the selected popcounts gives every
// word its output offset.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // -0.0 ranks as +0.0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return max(u, 1u);  // 0 marks "no key" (only one negative NaN pattern is moved, to 1)
}

// Radix schedule of the selection, most significant digit first: a 4-bit digit (bits
// 31..28) counted on lane-private LDS columns, where every key takes part and same-digit
// keys must not pile onto one address, then digits of 11, 11 and 6 bits counted in a
// 2048-bin histogram, where only the keys still in play are spread over the bins.
constexpr int kBins = 2048;
__device__ __forceinline__ int radix_shift(int pass) { return pass == 1 ? 17 : (pass == 2 ? 6 : 0); }
__device__ __forceinline__ int radix_width(int pass) { return pass == 3 ? 6 : 11; }

// Lowest set lane of a ballot.  The digit searches always have one (the bins hold at least
// the keys still needed); an empty ballot gives lane 63, whose bins are in range.
__device__ __forceinline__ int first_lane(unsigned long long b) {
  return b ? __builtin_ctzll(b) : 63;
}

// Histogram bin of a key in a radix pass: its digit at `shift` when the key carries the
// digits chosen so far (prefix; its bits at and below the digit are 0), else `spare`, a bin
// nobody reads.  (key ^ prefix) >> shift keeps set bits above the digit exactly for keys
// outside the prefix.
__device__ __forceinline__ uint32_t radix_bin(uint32_t key, uint32_t prefix, int shift, int width,
                                              uint32_t spare) {
  const uint32_t u = (key ^ prefix) >> shift;
  return u < (1u << width) ? u : spare;
}

// Inclusive prefix sum over the wave's 64 lanes with DPP moves (no LDS round trips): a
// Hillis-Steele scan inside each row of 16 lanes (source lanes outside the row read 0), then
// rows 1 and 3 add the last lane of the row before and rows 2 and 3 the last lane of row 1.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

// Block-wide exclusive prefix sum of v over threads in tid order; *total = block sum.  One
// barrier: a caller alternates between two wsum buffers, so that a buffer is rewritten only
// after a later scan's barrier, by which time every thread has read it.
template <int NT>
__device__ __forceinline__ int block_scan_excl(int v, int* total, int* wsum) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = wsum[w];
    before += (w < wave) ? c : 0;
    all += c;
  }
  *total = all;
  return before + incl - v;
}

// v_writelane: lane `lane` of `old` replaced by the wave-uniform `src` (the LLVM intrinsic,
// declared by name; the compiler inserts the wait states its SGPR operands need)
extern "C" __device__ int lane_write(int src, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

constexpr int kSegIdx = 32768;          // indices per compaction segment
constexpr int kSegWords = kSegIdx / 32;  // bitmap words per segment

template <int NT, int KPT>
__global__ void __launch_bounds__(NT) topk_radix(const float* __restrict__ scores,
                                                 const int* __restrict__ q_pos0,
                                                 const int* __restrict__ n_pool,
                                                 int* __restrict__ topk_idx,
                                                 float* __restrict__ topk_score, int T, int N_cap,
                                                 int m, int k) {
  constexpr int NW = NT / 64;
  static_assert(kSegIdx % NT == 0 && NT % 64 == 0, "segment = whole block strides");
  static_assert(KPT * NT <= kSegIdx, "register keys must fit the first segment");
  static_assert(2 * KPT <= 64, "a wave's bitmap words of the register strides: one per lane");
  // two histograms used in alternate passes: kBins digit bins, then one spare bin per lane
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][kBins + 64];
  __shared__ uint32_t gtbits[kSegWords], eqbits[kSegWords];
  __shared__ __attribute__((aligned(16))) int wtot[NW];
  __shared__ __attribute__((aligned(16))) int tot[16];
  __shared__ int wsum[2][NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qrow = blockIdx.x;
  const int b = qrow / T, t = qrow % T;
  const int V = visible_entries(q_pos0, n_pool, b, t, m, N_cap);
  const float* s = scores + static_cast<size_t>(qrow) * N_cap;
  int* out_i = topk_idx + static_cast<size_t>(qrow) * k;
  float* out_s = topk_score ? topk_score + static_cast<size_t>(qrow) * k : nullptr;
  const int kk = min(k, V);

  if (kk == V) {  // every visible entry, in index order
    for (int p = tid; p < k; p += NT) {
      out_i[p] = p < V ? p : -1;
      if (out_s) out_s[p] = p < V ? s[p] : 0.f;
    }
    return;
  }

  // keys of this thread: index j*NT + tid; 0 for indices >= V (discounted, never selected).
  // All loads are issued before any is converted (indices clamped to the last key, in
  // bounds): with the load and its use in one step, every key waited a memory round trip.
  const int n_strides = (V + NT - 1) / NT;
  uint32_t key[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    key[j] = j < n_strides ? __float_as_uint(s[min(j * NT + tid, V - 1)]) : 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    key[j] = (j < n_strides && j * NT + tid < V) ? score_key(__uint_as_float(key[j])) : 0u;

  // strides past the row are skipped (block-uniform); the last one may hold empty slots
  const int n_reg = min(n_strides, KPT);
  const int n_inv = n_reg * NT - min(V, n_reg * NT);
  for (int i = tid; i < 2 * (kBins + 64); i += NT) (&hist[0][0])[i] = 0;
  __syncthreads();

  // Thread t owns the BPT bins kBins - BPT(t+1) .. kBins - BPT t - 1: in thread order the
  // bins run from the highest digit down, so a block scan of the threads' bin sums gives
  // the count of keys at or above each thread's bins.
  constexpr int BPT = kBins / NT;
  static_assert(BPT * NT == kBins && BPT <= 8, "bins per thread");
  uint32_t prefix = 0, mask = 0;
  int remaining = kk;
  bool done = false;
  {  // first digit: bits 31..28 on lane-private columns, [digit][lane] in hist[0]
    uint32_t* hcol = &hist[0][lane];
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < n_reg) atomicAdd(hcol + (key[j] >> 28) * 64, 1u);
    for (int j = KPT; j < n_strides; ++j) {
      const int i = j * NT + tid;
      if (i >= V) break;
      atomicAdd(hcol + (score_key(s[i]) >> 28) * 64, 1u);
    }
    __syncthreads();
#pragma unroll
    for (int d = wave; d < 16; d += NW) {
      const int c = wave_sum(static_cast<int>(hist[0][d * 64 + lane]));
      // the n_inv empty register slots hold key 0: digit 0
      if (lane == 0) tot[d] = c - (d == 0 ? n_inv : 0);
    }
    __syncthreads();
    int tv[16];  // every thread derives the digit from the 16 totals, read at once
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int4 x = reinterpret_cast<const int4*>(tot)[q];
      tv[4 * q] = x.x; tv[4 * q + 1] = x.y; tv[4 * q + 2] = x.z; tv[4 * q + 3] = x.w;
    }
    int above = 0, digit = 0, in_digit = 0;
    bool found = false;
#pragma unroll
    for (int d = 15; d >= 0; --d) {
      const int c = tv[d];
      if (!found && above + c >= remaining) { digit = d; in_digit = c; found = true; }
      if (!found) above += c;
    }
    remaining -= above;
    prefix = static_cast<uint32_t>(digit) << 28;
    mask = 0xF0000000u;
    done = in_digit == remaining;
  }
  // passes 1..3 in hist[1], hist[0], hist[1]: hist[0]'s columns are cleared in pass 1
#pragma unroll 1
  for (int pass = 1; pass < 4 && !done; ++pass) {
    const int shift = radix_shift(pass), width = radix_width(pass);
    uint32_t* h = hist[pass & 1];
    const uint32_t spare = kBins + lane;  // keys outside the prefix: a lane-private bin
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < n_reg) atomicAdd(h + radix_bin(key[j], prefix, shift, width, spare), 1u);
    for (int j = KPT; j < n_strides; ++j) {
      const int i = j * NT + tid;
      if (i >= V) break;
      atomicAdd(h + radix_bin(score_key(s[i]), prefix, shift, width, spare), 1u);
    }
    __syncthreads();
    // this thread's bins (and the other histogram's, cleared for the next pass: its last
    // readers finished before the barrier above, its next writers come after the next)
    const int b0 = kBins - BPT * (tid + 1);
    int mine = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      mine += static_cast<int>(h[b0 + i]);
      hist[(pass + 1) & 1][b0 + i] = 0;
    }
    // the n_inv empty register slots hold key 0: bin 0 while the prefix is all zeros
    if (b0 == 0 && prefix == 0u) mine -= n_inv;
    const int incl = wave_incl_scan(mine);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    // the wave whose bins hold the remaining-th key from the top, then (every wave alike)
    // the thread within it and the bin within that thread
    int above = 0, ws = 0;
    bool found = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = wtot[w];
      if (!found && above + c >= remaining) { ws = w; found = true; }
      if (!found) above += c;
    }
    const int bw = kBins - BPT * (64 * ws + lane + 1);  // the bins of thread 64 ws + lane
    int v[BPT], lsum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      v[i] = static_cast<int>(h[bw + i]);
      if (bw + i == 0 && prefix == 0u) v[i] -= n_inv;
      lsum += v[i];
    }
    const int lincl = wave_incl_scan(lsum);
    const unsigned long long hit = __ballot(above + lincl >= remaining);
    const int L = first_lane(hit);
    above += __builtin_amdgcn_readlane(lincl - lsum, L);
    int digit = 0, in_digit = 0;
    found = false;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {  // the lane's bins from the highest down
      const int c = __builtin_amdgcn_readlane(v[i], L);
      if (!found && above + c >= remaining) { digit = bw + i; in_digit = c; found = true; }
      if (!found) above += c;
    }
    digit = __builtin_amdgcn_readlane(digit, L);  // bw differs per lane: take lane L's
    remaining -= above;
    prefix |= static_cast<uint32_t>(digit) << shift;
    mask |= ((1u << width) - 1u) << shift;
    done = in_digit == remaining;  // the whole bucket is taken: threshold found
  }

  // index-ordered compaction; equal keys (under mask) taken lowest index first
  int eq_base = 0, out_base = 0;
  for (int seg0 = 0; seg0 < V; seg0 += kSegIdx) {
    const int seg_end = min(V, seg0 + kSegIdx);
    const int j0 = seg0 / NT, j1 = (seg_end + NT - 1) / NT;
    if (seg0 == 0) {  // register keys all lie in the first segment (KPT * NT <= kSegIdx)
      int gw = 0, ew = 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const bool ok = key[j] != 0u;
        const uint32_t km = key[j] & mask;
        const unsigned long long g = __ballot(ok && km > prefix);
        const unsigned long long e = __ballot(ok && km == prefix);
        gw = lane_write(static_cast<int>(g), 2 * j, gw);
        gw = lane_write(static_cast<int>(g >> 32), 2 * j + 1, gw);
        ew = lane_write(static_cast<int>(e), 2 * j, ew);
        ew = lane_write(static_cast<int>(e >> 32), 2 * j + 1, ew);
      }
      if (lane < 2 * KPT) {
        const int w = (lane >> 1) * (NT / 32) + wave * 2 + (lane & 1);
        gtbits[w] = static_cast<uint32_t>(gw);
        eqbits[w] = static_cast<uint32_t>(ew);
      }
    }
    for (int j = max(j0, KPT); j < j1; ++j) {
      const bool ok = j * NT + tid < V;
      const uint32_t km = ok ? (score_key(s[j * NT + tid]) & mask) : 0u;
      const unsigned long long g = __ballot(ok && km > prefix);
      const unsigned long long e = __ballot(ok && km == prefix);
      if (lane < 2) {
        const int w = (j * NT + wave * 64 - seg0) / 32 + lane;
        gtbits[w] = static_cast<uint32_t>(lane ? g >> 32 : g);
        eqbits[w] = static_cast<uint32_t>(lane ? e >> 32 : e);
      }
    }
    __syncthreads();
    // each thread owns WPT consecutive words of the segment
    constexpr int WPT = kSegWords / NT > 0 ? kSegWords / NT : 1;
    const int n_words = (seg_end - seg0 + 31) / 32;
    const int w0 = tid * WPT;
    int eq_cnt = 0;
#pragma unroll
    for (int q = 0; q < WPT; ++q)
      if (w0 + q < n_words) eq_cnt += __popc(eqbits[w0 + q]);
    int eq_tot;
    int eq_pre = eq_base + block_scan_excl<NT>(eq_cnt, &eq_tot, wsum[0]);
    uint32_t sel[WPT];
    int sel_cnt = 0;
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      sel[q] = 0;
      if (w0 + q < n_words) {
        uint32_t e = eqbits[w0 + q];
        const int allow = remaining - eq_pre;  // equal keys still to take
        const int pe = __popc(e);
        eq_pre += pe;
        if (allow <= 0) {
          e = 0;
        } else {
          for (int c = pe; c > allow; --c) e &= ~(1u << (31 - __clz(e)));  // drop highest
        }
        sel[q] = gtbits[w0 + q] | e;
        sel_cnt += __popc(sel[q]);
      }
    }
    int sel_tot;
    int pos = out_base + block_scan_excl<NT>(sel_cnt, &sel_tot, wsum[1]);
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      uint32_t w = sel[q];
      while (w) {
        const int bit = __ffs(w) - 1;
        w &= w - 1;
        const int i = seg0 + (w0 + q) * 32 + bit;
        if (pos < k) {
          out_i[pos] = i;
          if (out_s) out_s[pos] = s[i];
        }
        ++pos;
      }
    }
    eq_base += eq_tot;
    out_base += sel_tot;
    // every bitmap read came before the barrier of the second scan: the next segment may
    // rebuild them
  }
  for (int p = kk + tid; p < k; p += NT) {
    out_i[p] = -1;
    if (out_s) out_s[p] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Top-k for many short rows (prefill): one wave per row, four rows per block, no block
// barriers.  Same selection as topk_radix (a 4-bit digit on lane-private columns, summed by
// 4-lane quads, then 11-, 11- and 6-bit digits on a per-wave 2048-bin histogram: lane l
// holds 32 bins, the highest first, a wave scan finds the lane and a second one the bin;
// early exit), and the compaction walks the row once in index order, 64 keys per ballot,
// carrying the running counts of selected and of equal keys (ties to the lower entry
// index).
// Keys of lane l: indices j*64 + l; the first KPL strides stay in registers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_wave_sync() {
  // all LDS operations of this wave done before the next ones are issued
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// The score a key encodes (inverse of score_key; a score of -0.0 comes back as +0.0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ int quad_sum(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  return x;
}

template <int KPL>
__global__ void __launch_bounds__(256) topk_wave(const float* __restrict__ scores,
                                                 const int* __restrict__ q_pos0,
                                                 const int* __restrict__ n_pool,
                                                 int* __restrict__ topk_idx,
                                                 float* __restrict__ topk_score, int rows, int T,
                                                 int N_cap, int m, int k) {
  // per wave: kBins digit bins, then one spare bin per lane (keys outside the prefix); the
  // first digit's [16][64] lane columns use the first 1024 bins
  __shared__ __attribute__((aligned(16))) uint32_t hist[4][kBins + 64];
  __shared__ __attribute__((aligned(16))) int tots[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;  // wave-uniform; the kernel has no block barrier
  const int b = row / T, t = row % T;
  const int V = visible_entries(q_pos0, n_pool, b, t, m, N_cap);
  const float* s = scores + static_cast<size_t>(row) * N_cap;
  int* out_i = topk_idx + static_cast<size_t>(row) * k;
  float* out_s = topk_score ? topk_score + static_cast<size_t>(row) * k : nullptr;
  const int kk = min(k, V);

  if (kk == V) {
    for (int p = lane; p < k; p += 64) {
      out_i[p] = p < V ? p : -1;
      if (out_s) out_s[p] = p < V ? s[p] : 0.f;
    }
    return;
  }

  const int n_str = (V + 63) / 64;
  uint32_t key[KPL];  // loads issued together (clamped in bounds), then converted
#pragma unroll
  for (int j = 0; j < KPL; ++j) key[j] = j < n_str ? __float_as_uint(s[min(j * 64 + lane, V - 1)]) : 0u;
#pragma unroll
  for (int j = 0; j < KPL; ++j)
    key[j] = (j < n_str && j * 64 + lane < V) ? score_key(__uint_as_float(key[j])) : 0u;
  const int n_reg = min(n_str, KPL);  // register strides in use (wave-uniform)
  const int n_inv = n_reg * 64 - min(V, n_reg * 64);

  // Lane l owns the 32 bins lb .. lb + 31, lb = kBins - 32(l+1): in lane order the bins run
  // from the highest digit down, so a wave scan of the lanes' sums counts the keys at or
  // above each lane's bins.
  uint32_t* hw = hist[wave];
  const int lb = kBins - 32 * (lane + 1);
#pragma unroll
  for (int v = 0; v < 8; ++v) *reinterpret_cast<uint4*>(hw + lb + 4 * v) = make_uint4(0, 0, 0, 0);

  uint32_t prefix = 0, mask = 0;
  int remaining = kk;
  bool done = false;
  {  // first digit: bits 31..28 on lane-private columns hw[digit * 64 + lane]
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (j < n_reg) atomicAdd(hw + (key[j] >> 28) * 64 + lane, 1u);
    for (int j = KPL; j < n_str; ++j) {
      const int i = j * 64 + lane;
      if (i < V) atomicAdd(hw + (score_key(s[i]) >> 28) * 64 + lane, 1u);
    }
    lds_wave_sync();
    // lane 4d + q sums columns 16q .. 16q + 15 of digit d and clears them
    const int rd = lane >> 2, rq = lane & 3;
    uint4* rsum = reinterpret_cast<uint4*>(hw + rd * 64 + rq * 16);
    int c = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 h = rsum[v];
      c += static_cast<int>(h.x + h.y + h.z + h.w);
      rsum[v] = make_uint4(0, 0, 0, 0);
    }
    c = quad_sum(c);
    if (rd == 0) c -= n_inv;  // empty register slots (key 0)
    if (rq == 0) tots[wave][rd] = c;
    lds_wave_sync();
    int tv[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int4 q4 = reinterpret_cast<const int4*>(&tots[wave][0])[v];
      tv[4 * v] = q4.x; tv[4 * v + 1] = q4.y; tv[4 * v + 2] = q4.z; tv[4 * v + 3] = q4.w;
    }
    int above = 0, digit = 0, in_digit = 0;
    bool found = false;
#pragma unroll
    for (int d = 15; d >= 0; --d) {
      if (!found) {
        if (above + tv[d] >= remaining) { digit = d; in_digit = tv[d]; found = true; }
        else above += tv[d];
      }
    }
    remaining -= above;
    prefix = static_cast<uint32_t>(digit) << 28;
    mask = 0xF0000000u;
    done = in_digit == remaining;
  }
#pragma unroll 1
  for (int pass = 1; pass < 4 && !done; ++pass) {
    const int shift = radix_shift(pass), width = radix_width(pass);
    const uint32_t spare = kBins + lane;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (j < n_reg) atomicAdd(hw + radix_bin(key[j], prefix, shift, width, spare), 1u);
    for (int j = KPL; j < n_str; ++j) {
      const int i = j * 64 + lane;
      if (i < V) atomicAdd(hw + radix_bin(score_key(s[i]), prefix, shift, width, spare), 1u);
    }
    lds_wave_sync();
    int lsum = 0;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const uint4 x = *reinterpret_cast<const uint4*>(hw + lb + 4 * v);
      lsum += static_cast<int>(x.x + x.y + x.z + x.w);
    }
    // the n_inv empty register slots hold key 0: bin 0 while the prefix is all zeros
    if (lb == 0 && prefix == 0u) lsum -= n_inv;
    const int incl = wave_incl_scan(lsum);
    const int L = first_lane(__ballot(incl >= remaining));  // the lane holding the key
    int above = __builtin_amdgcn_readlane(incl - lsum, L);
    // lane L's bins from the highest down: lane i < 32 takes bin top - i
    const int top = kBins - 32 * L - 1;
    int c = 0;
    if (lane < 32) {
      c = static_cast<int>(hw[top - lane]);
      if (top - lane == 0 && prefix == 0u) c -= n_inv;
    }
    const int cincl = wave_incl_scan(c);
    const int I = min(first_lane(__ballot(lane < 32 && above + cincl >= remaining)), 31);
    const int digit = top - I;
    const int in_digit = __builtin_amdgcn_readlane(c, I);
    above += __builtin_amdgcn_readlane(cincl - c, I);
    // clear the bins for the next pass (after the reads above: one wave, LDS in order)
#pragma unroll
    for (int v = 0; v < 8; ++v) *reinterpret_cast<uint4*>(hw + lb + 4 * v) = make_uint4(0, 0, 0, 0);
    remaining -= above;
    prefix |= static_cast<uint32_t>(digit) << shift;
    mask |= ((1u << width) - 1u) << shift;
    done = in_digit == remaining;
    lds_wave_sync();
  }

  // one index-ordered walk over the row
  const unsigned long long below = (1ull << lane) - 1ull;
  int eq_seen = 0, out_pos = 0;
  auto emit = [&](int i, bool ok, uint32_t kj) {
    const uint32_t km = kj & mask;
    const bool gt = ok && km > prefix;
    const bool eq = ok && km == prefix;
    const unsigned long long eb = __ballot(eq);
    const bool sel = gt || (eq && eq_seen + __popcll(eb & below) < remaining);
    eq_seen += __popcll(eb);
    const unsigned long long sb = __ballot(sel);
    const int pos = out_pos + __popcll(sb & below);
    if (sel && pos < k) {  // exactly kk keys are selected; the bound only guards the buffer
      out_i[pos] = i;
      if (out_s) out_s[pos] = key_score(kj);  // from the key: no reload of the row
    }
    out_pos += __popcll(sb);
  };
  // the search ended on a whole bucket: every key at or above the prefix is kept (a key
  // compares with the prefix as its masked value does, the prefix being zero below the mask)
  auto emit_ge = [&](int i, bool ok, uint32_t kj) {
    const bool sel = ok && kj >= prefix;
    const unsigned long long sb = __ballot(sel);
    const int pos = out_pos + __popcll(sb & below);
    if (sel && pos < k) {
      out_i[pos] = i;
      if (out_s) out_s[pos] = key_score(kj);
    }
    out_pos += __popcll(sb);
  };
  auto walk = [&](auto&& f) {
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (j < n_str) f(j * 64 + lane, key[j] != 0u, key[j]);
    for (int j = KPL; j < n_str; ++j) {
      const int i = j * 64 + lane;
      const bool ok = i < V;
      f(i, ok, ok ? score_key(s[i]) : 0u);
    }
  };
  if (done) walk(emit_ge);
  else walk(emit);
  for (int p = kk + lane; p < k; p += 64) {
    out_i[p] = -1;
    if (out_s) out_s[p] = 0.f;
  }
}

hipError_t launch_topk(const float* scores, const int* q_pos0, const int* n_pool, int* topk_idx,
                       float* topk_score, int B, int T, int N_cap, int m, int k, hipStream_t st) {
  if (B == 0 || T == 0) return hipSuccess;
  const int rows = B * T;
  if (N_cap > 8192 && rows < 2048) {
    // few long rows (decode): one block of 1024 threads per row
    hipLaunchKernelGGL((topk_radix<1024, 32>), dim3(rows), dim3(1024), 0, st, scores, q_pos0,
                       n_pool, topk_idx, topk_score, T, N_cap, m, k);
  } else {
    const dim3 grid(div_up(rows, 4));
    if (N_cap <= 2048)
      hipLaunchKernelGGL((topk_wave<32>), grid, dim3(256), 0, st, scores, q_pos0, n_pool,
                         topk_idx, topk_score, rows, T, N_cap, m, k);
    else if (N_cap <= 4096)
      hipLaunchKernelGGL((topk_wave<64>), grid, dim3(256), 0, st, scores, q_pos0, n_pool,
                         topk_idx, topk_score, rows, T, N_cap, m, k);
    else if (N_cap <= 8192)  // rows of up to 8192 keys: one block of 256 threads, 32 keys a thread
      hipLaunchKernelGGL((topk_radix<256, 32>), dim3(rows), dim3(256), 0, st, scores, q_pos0,
                         n_pool, topk_idx, topk_score, T, N_cap, m, k);
    else  // strides past the 64 in registers are re-read from the score row on every pass
      hipLaunchKernelGGL((topk_wave<64>), grid, dim3(256), 0, st, scores, q_pos0, n_pool,
                         topk_idx, topk_score, rows, T, N_cap, m, k);
  }
  return hipGetLastError();
}

}  // namespace dsv4
