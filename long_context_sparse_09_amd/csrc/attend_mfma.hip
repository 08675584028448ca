// Shared-K=V multi-query attention on MFMA for gfx950 (bf16 storage, fp32 accumulation),
// 64 query heads x head_dim 512: the CSA gather-then-attend and the HCA / sliding dense-range
// attend share this kernel.
//
// Source: DeepSeek-V4 model page (Transformers docs), "Hybrid attention (§2.3)": one K=V head
// (num_key_value_heads = 1) read as both key and value, partial RoPE on the trailing
// qk_rope_head_dim channels, the output rope slice rotated at position -i (eq. 26), a per-head
// learnable sink (eq. 27), and the sliding-window K=V branch concatenated before the
// compressed keys.  "Attention mask layout": sliding window cut, CSA -1 sentinel, HCA entry
// visibility w < (t+1)//m.
//
// Work decomposition
//   * Persistent workgroups (one per CU) walk their queries as one stream of 32-key tiles:
//     the window rows of a query, then its selected (CSA) or visible (HCA) pool rows.
//   * Ten wavefronts in three roles, pipelined by one tile.  Wave w runs on SIMD w mod 4;
//     each SIMD carries one score and one value wave (and SIMDs 0, 1 a gather wave), so the
//     softmax and epilogue work of one role overlaps the matrix work of the other:
//       - gather (waves 8, 9: rows 0..15 and 16..31): move each tile's 32 key rows (1 KB
//         each) from global memory straight into LDS (buffer_load ... lds, one row
//         descriptor per row), three tiles ahead, into a ring of four tile buffers.  A
//         vector-memory issue stalls the issuing wave at the CU's fill rate, so the gather
//         sits in its own waves; for CSA they also copy the next query's index list into
//         LDS while the current query's tiles stream, so a query switch waits on nothing;
//       - score (waves 0..3 = hq): heads [16hq, 16hq+16), all 512 channels.  S^T = K . Q^T
//         on v_mfma_f32_16x16x32_bf16 (A = 16 key rows from LDS, B = the rotated Q in
//         registers; two 16-key blocks x 16 channel steps), then the online softmax of the
//         tile; publishes P (bf16, [head][key] rows) and the rescale factor of the running
//         max;
//       - value (waves 4..7 = kq): O^T[channels 128kq .. +128, all 64 heads] += V^T . P^T
//         on v_mfma_f32_32x32x16_bf16, with V^T read from the same row-major tile through
//         ds_read_tr16_b64 (K = V is stored once); each V^T fragment serves both 32-head
//         blocks.
//     In step s the score waves work on tile s+1, the value waves on tile s and the gather
//     waves fill tile s+3.  Per tile each SIMD runs 32 16x16x32 and 16 32x32x16 matrix
//     instructions (1024 cycles).  One workgroup barrier per step: tile s+1 landed, P(s)
//     published, the buffer of tile s-1 free.
//   * Online softmax in the log2 domain; the running max moves only when a logit exceeds it
//     by 2^8 (lazy rescale).  The state starts from the sink: max = s_h, sum = 1, value 0.
//   * RoPE angles are formed per lane in double precision (position x frequency, reduced to
//     turns) and fed to the hardware sin / cos, for the Q rotation and the output
//     counter-rotation alike.
//   * LDS rows are 1024 B with their 16-byte chunks XOR-swizzled per row (chunk c of row r
//     sits at c ^ f(r), f(r) = 4(r mod 4) + ((r >> 2) mod 4)), so the 16-row b128 reads of
//     QK^T and the 4-row transposing reads of PV each touch 64 distinct banks.
//   * Query order: heaviest first, and each round hands G/8 consecutive queries to the G/8
//     workgroups of one XCD, so the window rows that neighbouring queries share are fetched
//     into that XCD's L2 once.  Q is loaded and the output stored non-temporally.
#include "common.h"
#include "launch.h"

namespace dsv4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

namespace {

constexpr int AH = 64;                     // query heads
constexpr int AD = 512;                    // head_dim
constexpr int ANK = 32;                    // keys per tile
constexpr int APITCH = AD * 2;             // LDS bytes per key row (swizzled, no pad)
constexpr int ATILE = ANK * APITCH;        // bytes per tile buffer
constexpr int NSLOT = 4;                   // tile ring
constexpr int PPITCH = ANK * 2 + 16;      // bytes per head row of a P tile (32 keys, padded)
constexpr int P_OFF = NSLOT * ATILE;       // P tiles: [parity][64 heads][32 keys] bf16
constexpr int AL_OFF = P_OFF + 2 * AH * PPITCH;      // rescale factors: [parity][64 heads]
constexpr int LS_OFF = AL_OFF + 2 * 64 * 4;          // softmax sums at a query's end: [parity][64]
constexpr int KL_OFF = LS_OFF + 2 * 64 * 4;          // gather waves' key lists (CSA) [parity]
constexpr int kMaxTopk = 1024;                       // key-list capacity on this path
constexpr int RL_OFF = KL_OFF + 2 * kMaxTopk * 4;    // raw index list of the next query [gather wave]
constexpr int NK_OFF = RL_OFF + 2 * kMaxTopk * 4;    // key counts of queries [j % 8]
constexpr int RT_OFF = NK_OFF + 8 * 4;               // RoPE (cos, sin) of queries [j % 8][32 pairs]
constexpr int kLdsBytes = RT_OFF + 8 * 32 * 8;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
constexpr float kLazy = 8.f;               // log2-domain headroom before the running max moves
constexpr double kInv2Pi = 0.15915494309189533576888376337251;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

// LDS row swizzle: 16-byte chunk c of key row r sits at chunk c ^ swz(r).  swz is a
// bijection on every 16 aligned rows (the 16 lanes of a b128 read of QK^T hit 16 different
// bank groups) and, on every 4 aligned rows, differs in bits 2-3 only (the 4 rows x 4
// chunks of a transposing read of PV hit 16 different bank groups too).
__device__ __forceinline__ int swz(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }

// Buffer resources: global memory is read and written through buffer instructions (SGPR
// descriptor + SGPR offset + one 32-bit VGPR lane offset).  A memory instruction that takes
// a 64-bit VGPR address per lane issues far more slowly while other waves on the SIMD keep
// the matrix core busy; the buffer form does not.  Reads past num_records return zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer
constexpr unsigned kOutOfRange = 0xFFFFF000u;  // row offset beyond every descriptor: reads zeros
__device__ __forceinline__ rsrc_t make_rs(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}
constexpr int kNT = 2;  // cache policy bits of the buffer instructions: non-temporal

// Partner value across the two 32-lane halves (lane l <-> lane l ^ 32), combined.
__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Partner value across the 16-lane rows of each 32-lane half (lane l <-> lane l ^ 16), combined.
__device__ __forceinline__ float xrow_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xrow_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// cos / sin of angle (pos * inv_freq) for one rotary pair: the product is reduced to turns in
// double precision, the hardware sin / cos take turns.
__device__ __forceinline__ void rope_pair(double pos, double inv_freq, float& c, float& s) {
  const double turns = pos * inv_freq * kInv2Pi;
  const float frac = static_cast<float>(turns - rint(turns));
  c = __builtin_amdgcn_cosf(frac);
  s = __builtin_amdgcn_sinf(frac);
}

// Workgroup barrier for LDS hand-offs.  __syncthreads() also drains every outstanding
// vector-memory operation of the calling wave (its release fence waits for vmcnt 0), which
// would make a gather wave wait for tiles it has only just issued; here only this wave's
// LDS operations are drained.  The gather waves order their tiles with explicit vmcnt waits.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left open
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// This lane's id, recomputed where it is used (two instructions) rather than kept live: the
// optimiser cannot hoist it, so offsets derived from it are not held in registers (or
// spilled) across the tile loop.
__device__ __forceinline__ int lane_now() {
  int l = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(l));
  return l;
}

// Per-query description, computed identically by every wave that needs it.
// A work item is one query, or one of n_split key ranges of a query (split mode): tiles
// tb .. tb + n_tiles - 1 of the query's keys.
struct QInfo {
  int b, t, r0, n_win, n_keys, n_tiles, tb, sp;
  long long p;
};

}  // namespace

// Load of a value every lane reads at the same address, through the constant address space:
// a scalar load, which neither waits for nor is waited on by vector-memory traffic.
__device__ __forceinline__ int load_uniform(const int* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) int*>(reinterpret_cast<uintptr_t>(p));
}

// Every field is uniform across the wave; keep it in scalar registers.
__device__ __forceinline__ QInfo uniform(const QInfo& d) {
  QInfo u;
  u.b = __builtin_amdgcn_readfirstlane(d.b);
  u.t = __builtin_amdgcn_readfirstlane(d.t);
  u.r0 = __builtin_amdgcn_readfirstlane(d.r0);
  u.n_win = __builtin_amdgcn_readfirstlane(d.n_win);
  u.n_keys = __builtin_amdgcn_readfirstlane(d.n_keys);
  u.n_tiles = __builtin_amdgcn_readfirstlane(d.n_tiles);
  u.tb = __builtin_amdgcn_readfirstlane(d.tb);
  u.sp = __builtin_amdgcn_readfirstlane(d.sp);
  const unsigned long long pu = static_cast<unsigned long long>(d.p);
  u.p = static_cast<long long>((static_cast<unsigned long long>(__builtin_amdgcn_readfirstlane(static_cast<unsigned>(pu >> 32))) << 32) |
                               __builtin_amdgcn_readfirstlane(static_cast<unsigned>(pu)));
  return u;
}

// Tile range of a work item.  The query's keys fill nq = max(1, ceil(n_keys / 32)) tiles (an
// empty query still runs one masked tile); split sp of n takes tiles [nq sp / n, nq (sp+1) / n),
// or, when that is empty, one fully masked tile (index nq) so that every item runs a step.
__device__ __forceinline__ void set_range(QInfo& d, int n_split) {
  const int nq = max(1, (d.n_keys + ANK - 1) / ANK);
  const int t0 = nq * d.sp / n_split, t1 = nq * (d.sp + 1) / n_split;
  d.tb = t1 > t0 ? t0 : nq;
  d.n_tiles = t1 > t0 ? t1 - t0 : 1;
}

// Position, window rows and (HCA) visible pool entries of the query of work item `item`;
// for CSA, n_keys and the tile range are completed by set_keys() once the compressed-key
// count is known.
template <bool CSA>
__device__ __forceinline__ QInfo query_geom(const AttendArgs& a, int item) {
  QInfo d;
  const int qid = item / a.n_split;
  d.sp = item - qid * a.n_split;
  d.b = qid / a.T;
  d.t = qid % a.T;
  d.p = static_cast<long long>(load_uniform(a.q_pos0 + d.b)) + d.t;
  const int kv0 = load_uniform(a.kv_pos0 + d.b);
  const long long lo = max(0LL, d.p - a.window + 1);
  d.r0 = static_cast<int>(max(lo - kv0, 0LL));
  const int r1 = static_cast<int>(min(d.p + 1 - kv0, static_cast<long long>(a.S_kv)));
  d.n_win = max(0, r1 - d.r0);
  d.n_keys = d.n_win;
  if constexpr (!CSA) {
    long long v = a.N_cap > 0 ? (d.p + 1) / a.m_hca : 0;
    v = min(v, static_cast<long long>(a.n_pool ? load_uniform(a.n_pool + d.b) : a.N_cap));
    v = min(v, static_cast<long long>(a.N_cap));
    d.n_keys += static_cast<int>(max(v, 0LL));
  }
  set_range(d, a.n_split);
  return uniform(d);
}

__device__ __forceinline__ void set_keys(QInfo& d, int n_cmp, int n_split) {
  d.n_keys = d.n_win + n_cmp;
  set_range(d, n_split);
}

template <bool CSA, int R>  // R = rotary channels, 0 or 64 (compile-time: only those chunks move)
__global__ void __attribute__((amdgpu_flat_work_group_size(640, 640), amdgpu_waves_per_eu(3, 3)))
attend_mfma_kernel(AttendArgs a) {
  static_assert(R == 0 || R == 64, "rotary width on this path");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: roles are per wave
  const int n_q = a.B * a.T * a.n_split;  // work items
  const int G = gridDim.x;
  const bf16_t* qbase = static_cast<const bf16_t*>(a.q);
  int* nk = reinterpret_cast<int*>(lds + NK_OFF);  // compressed-key counts of queries [j % 8]
  // (cos, sin) of each rotary pair's angle at a query's position, one row per query [j % 8]:
  // formed once by a gather wave when it starts the query, read by the score waves (Q
  // rotation) and the value waves (output counter-rotation, sine negated)
  float2* rt = reinterpret_cast<float2*>(lds + RT_OFF);

  // j-th query of this workgroup, as a rank in the heaviest-first order.  Workgroups are
  // dealt to the 8 XCDs round-robin; with G a multiple of 8, round j gives XCD x the ranks
  // [jG + xG/8, jG + (x+1)G/8), i.e. G/8 consecutive queries.
  const int g = static_cast<int>(blockIdx.x);
  const int slot = (G % 8) == 0 ? (g % 8) * (G / 8) + g / 8 : g;
  const int n_mine = (n_q - slot + G - 1) / G;
  auto qid_of = [&](int j) { return n_q - 1 - (j * G + slot); };

  if (wave >= 8) {
    // ------------------------------------------------------------------ gather waves
    // Wave 8 moves rows 0..15 of every tile, wave 9 rows 16..31; both walk the same cursor.
    __builtin_amdgcn_s_setprio(3);  // its issue slots go first: the other waves wait on its tiles
    const int gh = wave - 8;
    const bf16_t* win0 = static_cast<const bf16_t*>(a.kv_win);
    const bf16_t* pool0 = static_cast<const bf16_t*>(a.pool);
    int* kl = reinterpret_cast<int*>(lds + KL_OFF);  // [query parity][kMaxTopk]
    int iq = 0, it = 0;  // issue cursor: query rank, tile
    QInfo qi;
    // lane i < R/2: frequency of rotary pair i, loaded before any tile or list load is issued
    const double fq = lane < R / 2 ? a.inv_freq[lane] : 0.0;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    unsigned voff[16];  // lane offset of a row whose chunks are XOR-ed with j
#pragma unroll
    for (int j = 0; j < 16; ++j) voff[j] = static_cast<unsigned>(lane ^ j) << 4;
    // CSA: the raw index list of query j + 1 is copied into LDS (LDS-DMA) while query j is
    // gathered, so that switching queries waits on no memory latency.  The copy of query
    // j + 1 is issued before the tile loads of every later step, so once the loads of the
    // current tile are the only ones allowed in flight (vmcnt(16)) it has landed.
    constexpr int NC = kMaxTopk / 64;
    const int* rl = reinterpret_cast<const int*>(lds + RL_OFF) + gh * kMaxTopk;
    // 16-byte lane loads copy entries 0 .. k4-1 (k4 = k rounded down to a multiple of 4);
    // lanes at or past k4 are masked off, so no load straddles the end of the list (a load
    // crossing the descriptor's end may read as zeros, entry 0, for its valid entries too).
    // The k - k4 remaining entries move as one 4-byte load per lane, into slots no 16-byte
    // load writes.
    auto list_dma = [&](int j) {
      const QInfo d = query_geom<CSA>(a, qid_of(j));
      const int* row = a.topk_idx + (static_cast<size_t>(d.b) * a.T + d.t) * a.k;
      const int k4 = a.k & ~3;
      const rsrc_t idx_rs = make_rs(row, static_cast<unsigned>(a.k) * 4u);
#pragma unroll
      for (int c = 0; c < kMaxTopk / 256; ++c)  // 256 entries (1 KB) per instruction
        if (c * 256 < k4 && c * 256 + lane * 4 < k4)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(idx_rs, (lds_void*)(rl + c * 256), 16,
                                                   static_cast<unsigned>(c * 1024 + lane * 16), 0, 0, 0);
      if (k4 != a.k && lane < a.k - k4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(idx_rs, (lds_void*)(rl + k4), 4,
                                                 static_cast<unsigned>(k4 * 4 + lane * 4), 0, 0, 0);
    };
    if constexpr (CSA) list_dma(0);
    auto load_query = [&](int j) {
      qi = query_geom<CSA>(a, qid_of(j));
      if constexpr (CSA) {  // compact the valid entries, in order
        if (j == 0) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        else __builtin_amdgcn_s_waitcnt(0x4F70);         // vmcnt(16): all but this tile's loads
        int ld[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) ld[c] = c * 64 < a.k ? rl[c * 64 + lane] : -1;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): read before the next copy lands
        if (j + 1 < n_mine) list_dma(j + 1);
        int* klq = kl + (j & 1) * kMaxTopk;
        int base = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (c * 64 >= a.k) break;  // uniform
          const int i = c * 64 + lane;
          const int e = i < a.k ? ld[c] : -1;
          const bool v = e >= 0 && e < a.N_cap;
          const unsigned long long m = __ballot(v);
          const int pos = base + __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(m), 0));
          if (v) klq[pos] = e;
          base += __popcll(m);
        }
        set_keys(qi, base, a.n_split);
      }
      if (lane == 0) nk[j & 7] = qi.n_keys - qi.n_win;  // compressed keys of query j
      if (R > 0 && gh == 0 && lane < R / 2) {
        float c, sn;
        rope_pair(static_cast<double>(qi.p + a.pos_off), fq, c, sn);
        rt[(j & 7) * 32 + lane] = make_float2(c, sn);
      }
    };
    unsigned rlo = 0, rhi = 0;
    auto tile_addr = [&]() {  // lane l < 32: address of key (tb + it)*32 + l of item iq
      const int x = (qi.tb + it) * ANK + (lane & 31);
      const bf16_t* row;
      if (x < qi.n_keys) {
        if (x < qi.n_win) {
          row = win0 + (static_cast<size_t>(qi.b) * a.S_kv + qi.r0 + x) * AD;
        } else {
          const int e = CSA ? kl[(iq & 1) * kMaxTopk + x - qi.n_win] : x - qi.n_win;
          row = pool0 + (static_cast<size_t>(qi.b) * a.N_cap + e) * AD;
        }
      } else {  // masked filler: the query's own first row (in bounds, finite)
        row = qbase + (static_cast<size_t>(qi.b) * a.T + qi.t) * AH * AD;
      }
      const unsigned long long rp = reinterpret_cast<unsigned long long>(row);
      rlo = static_cast<unsigned>(rp);
      rhi = static_cast<unsigned>(rp >> 32);
    };
    auto issue_half = [&](int h, int sl) {  // rows 16h .. 16h + 15 into tile buffer sl
      unsigned char* tb = lds + sl * ATILE;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = h * 16 + i;
        const unsigned lo32 = __builtin_amdgcn_readlane(rlo, r);
        const unsigned hi32 = __builtin_amdgcn_readlane(rhi, r);
        void* src = reinterpret_cast<void*>((static_cast<unsigned long long>(hi32) << 32) | lo32);
        const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(src, static_cast<short>(0), APITCH, kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(tb + r * APITCH), 16, voff[swz(i)], 0, 0, 0);
      }
    };
    // this wave's rows, with the half a compile-time constant in each copy: the row address
    // then stays a scalar base plus one lane offset (the fast form of the load)
    auto issue_mine = [&](int sl) {
      if (gh == 0) issue_half(0, sl);
      else issue_half(1, sl);
    };
    int n_issued = 0;
    bool have = true;  // the issue cursor points at a tile
    auto advance = [&]() {
      ++n_issued;
      if (++it < qi.n_tiles) return;
      it = 0;
      if (++iq >= n_mine) {
        have = false;
        return;
      }
      load_query(iq);
    };

    load_query(0);
    // prologue: tiles 0 and 1 (16 row loads per tile from this wave)
    tile_addr();
    issue_mine(0);
    advance();
    if (have) {
      tile_addr();
      issue_mine(1);
      advance();
      __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16): tile 0 has landed
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    // step s: fill tile s + 3 (its buffer held tile s - 1), then wait for tile s + 2
    for (int s = -1;; ++s) {
      lds_barrier();  // X(s)
      if (have) {
        const int sl = n_issued % NSLOT;
        tile_addr();
        issue_mine(sl);
        advance();
        __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      if (!have && s + 1 >= n_issued) break;  // step n_tiles - 1 was the last
    }
    return;
  }

  float* alph = reinterpret_cast<float*>(lds + AL_OFF);  // [parity][64 heads]
  float* lsum = reinterpret_cast<float*>(lds + LS_OFF);  // [parity][64 heads]

  if (wave < 4) {
    // ------------------------------------------------------------------ score waves
    // Wave hq: heads [16hq, 16hq + 16), all channels.  S^T = K . Q^T per tile as two 16-key
    // blocks kb on v_mfma_f32_16x16x32_bf16: A = 16 key rows x 32 channels (LDS), B = 32
    // channels x 16 heads (registers).  Lane (h16, g4): head 16hq + h16; it holds keys
    // 16kb + 4g4 + v of that head and channels 32ks + 8g4 .. + 7 of its Q fragments.
    const int hq = wave;
    const int h16 = lane & 15, g4 = lane >> 4;
    const int head = hq * 16 + h16;
    constexpr int NKS = AD / 32;  // channel steps of 32
    const float c2 = a.scale * kLog2e;  // logits in the log2 domain
    const float sink2 = a.sink[head] * kLog2e;
    bf16x8_t qf[NKS];
    const unsigned qvoff = static_cast<unsigned>((head * AD + 8 * g4) * 2);
    auto load_q = [&](const QInfo& d) {
      const rsrc_t q_rs = make_rs(qbase + (static_cast<size_t>(d.b) * a.T + d.t) * AH * AD, AH * AD * 2);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(q_rs, qvoff + ks * 64, 0, kNT));
    };
    // rotary channels AD-R .. AD-1 = the last R/32 channel steps; this lane's pair i/2 of
    // step ks has index (32 ks + 8 g4 + i - (AD - R)) / 2
    auto rotate_q = [&](int j) {
      if (R == 0) return;
      const float2* tr = rt + (j & 7) * 32;
#pragma unroll
      for (int ks = NKS - R / 32; ks < NKS; ++ks) {
        const int pr0 = ((ks * 32 - (AD - R)) >> 1) + 4 * g4;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float2 cs = tr[pr0 + i / 2];
          const float c = cs.x, sn = cs.y;
          const float xv = static_cast<float>(qf[ks][i]), yv = static_cast<float>(qf[ks][i + 1]);
          qf[ks][i] = static_cast<__bf16>(xv * c - yv * sn);
          qf[ks][i + 1] = static_cast<__bf16>(xv * sn + yv * c);
        }
      }
    };
    // A operand (kb, ks): key row 16kb + h16, chunk 4ks + g4 at chunk (4ks + g4) ^ swz(h16):
    // byte kaddr0 + 16 KB kb, XOR 64 ks
    const int kaddr0 = h16 * APITCH + ((g4 ^ swz(h16)) << 4);
    // P row of this lane's head.  Within each 16-key block the key index has bits 2 and 3
    // swapped: a transposing V^T read gives lane (l32, half) keys 4half + 0..3 and
    // 8 + 4half + 0..3 of the block as its 8 B-operand values, so that these 8 keys sit in
    // 16 contiguous bytes.  Keys 16kb + 4g4 .. + 3 go to byte 2 (16kb + 4 swap(g4)).
    unsigned char* prow = lds + P_OFF + head * PPITCH + 8 * (((g4 & 1) << 1) | (g4 >> 1));

    int jq = 0, tq = 0;  // cursor: query rank, tile within it
    QInfo cq = query_geom<CSA>(a, qid_of(0));
    load_q(cq);
    float m_run = sink2, l_run = 1.f;
    for (int s = -1;; ++s) {
      lds_barrier();  // X(s): tile s + 1 has landed
      if (jq >= n_mine) break;  // this step would score tile s + 1
      if (tq == 0) {
        if constexpr (CSA) set_keys(cq, __builtin_amdgcn_readfirstlane(nk[jq & 7]), a.n_split);
        rotate_q(jq);
        m_run = sink2;
        l_run = 1.f;
      }
      const bool last = (tq + 1 == cq.n_tiles);
      const unsigned char* tb = lds + ((s + 1) % NSLOT) * ATILE;
      f32x4_t sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      constexpr int NI = 2 * NKS;  // matrix instructions per tile: i = 2 ks + kb
      constexpr int PF = 6;        // K fragments in flight
      bf16x8_t kr[PF];
      auto kfrag = [&](int i) {
        return *reinterpret_cast<const bf16x8_t*>(tb + ((kaddr0 + (i & 1) * (16 * APITCH)) ^ (64 * (i >> 1))));
      };
#pragma unroll
      for (int i = 0; i < PF; ++i) kr[i] = kfrag(i);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bf16x8_t kf = kr[i % PF];
        if (i + PF < NI) kr[i % PF] = kfrag(i + PF);
        sacc[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[i >> 1], sacc[i & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (last && jq + 1 < n_mine) load_q(query_geom<CSA>(a, qid_of(jq + 1)));  // next Q streams in
      // online softmax over the tile's 32 keys: this lane holds keys 16kb + 4g4 + v
      const int kbase = (cq.tb + tq) * ANK + 4 * g4;
      float sv[8];
      float tmax = -INFINITY;
      const bool ragged = (cq.tb + tq) * ANK + ANK > cq.n_keys;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kbase + (e >> 2) * 16 + (e & 3);
        sv[e] = (!ragged || key < cq.n_keys) ? sacc[e >> 2][e & 3] * c2 : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
      tmax = xrow_max(tmax);
      tmax = xhalf_max(tmax);
      const float m_new = (tmax > m_run + kLazy) ? tmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float psum = 0.f;
      float pe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pe[e] = __builtin_amdgcn_exp2f(sv[e] - m_new);
        psum += pe[e];
      }
      psum = xhalf_sum(xrow_sum(psum));
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const int par = (s + 1) & 1;
      unsigned char* pr = prow + par * (AH * PPITCH);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        *reinterpret_cast<u32x2_t*>(pr + 32 * kb) =
            u32x2_t{pack_bf16x2(pe[4 * kb], pe[4 * kb + 1]), pack_bf16x2(pe[4 * kb + 2], pe[4 * kb + 3])};
      if (g4 == 0) {
        alph[par * 64 + head] = alpha;
        if (last) lsum[par * 64 + head] = l_run;
      }
      if (a.n_split > 1 && last && g4 == 0) {
        // split mode: this key range's running max and sum (log2 domain, sink included)
        float* ml = a.part + static_cast<size_t>(n_q) * AH * AD + (static_cast<size_t>(qid_of(jq)) * AH + head) * 2;
        ml[0] = m_run;
        ml[1] = l_run;
      }
      if (last) {
        tq = 0;
        if (++jq < n_mine) cq = query_geom<CSA>(a, qid_of(jq));
      } else {
        ++tq;
      }
    }
    return;
  }

  // -------------------------------------------------------------------- value waves
  // Wave 4 + kq: output channels [128kq, 128kq + 128) of all 64 heads.  O^T[32 ch x 32 heads]
  // blocks (cb, hb) += V^T[32 ch x 16 keys] . P^T[16 keys x 32 heads] per 16-key half ks;
  // each V^T fragment serves both head blocks.  Lane (l32, half): head 32hb + l32, channels
  // 8q + 4half + j of each 32-channel block (q = 0..3).
  const int kq = wave - 4;
  const int half = lane >> 5, l32 = lane & 31;
  constexpr int NCB = 4;  // 32-channel blocks per wave
  // V^T transposing reads of channel block cb, key half ks: rows 16ks + 4half + i (lo) and
  // + 8 (hi), i = n16/4; channels 128kq + 32cb + 16dh + 4(n16%4), i.e. chunk 16kq + 4cb + j,
  // j = 2dh + (n16%4)/2.  With swz(row) = 4i + (half | 2hi) the chunk's bits 2-3 become
  // cb ^ i and bits 0-1 j ^ (half | 2hi): the byte offset is (tr_lo or tr_hi) ^ (64 cb),
  // plus 16 KB ks.
  int tr_lo, tr_hi;
  {
    const int n16 = lane & 15, dh = (lane >> 4) & 1;
    const int i = n16 >> 2, j = 2 * dh + ((n16 & 3) >> 1);
    const int common = 256 * kq + 64 * i + (n16 & 1) * 8;
    tr_lo = (4 * half + i) * APITCH + common + 16 * (j ^ half);
    tr_hi = (4 * half + i + 8) * APITCH + common + 16 * (j ^ (half | 2));
  }
  f32x16_t o[NCB][2];
  int jp = 0, tp = 0;  // cursor: query rank, tile within it
  QInfo cp = query_geom<CSA>(a, qid_of(0));
  // PV runs as one stream of 8 steps st = ks * NCB + cb (two matrix instructions each),
  // whose V fragments are read VPF steps ahead.
  constexpr int VPF = 2;
  bf16x8_t vr[VPF];
  auto vfrag = [&](const unsigned char* tb, int st) {
    const unsigned char* vb = tb + 16 * (st / NCB) * APITCH;
    // the XOR is formed at each read (volatile asm is not hoisted): keeping pre-XOR-ed
    // offsets live would push the accumulators out of registers
    const int x = 64 * (st % NCB);
    int olo, ohi;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(olo) : "v"(tr_lo), "s"(x));
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(ohi) : "v"(tr_hi), "s"(x));
    const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + olo));
    const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + ohi));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // epilogue of one query: normalise, counter-rotate (eq. 26), store.  A 32-lane swap pairs
  // the two 4-channel halves so that each lane writes 16 contiguous bytes.
  auto finish = [&](const QInfo& d, int j, const float (&inv)[2]) {
    const rsrc_t o_rs = make_rs(static_cast<bf16_t*>(a.out) + (static_cast<size_t>(d.b) * a.T + d.t) * AH * AD,
                                AH * AD * 2);
    // Lane-dependent offsets are formed here, from a fresh lane id: kept live across the
    // tile loop they were spilled, and each reload's wait (vmcnt) held the next store
    // behind every store before it.
    const int ln = lane_now();
    const int ob = ((ln & 31) * AD + 128 * kq + (ln >> 5) * 8) * 2;  // head block 0, channel block 0
    const float2* tr = reinterpret_cast<const float2*>(lds + RT_OFF + (j & 7) * 256 + (ln >> 5) * 16);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        // this lane's channels: cl0(g2) + 4 half + 0..3, cl0(g2) = 128kq + 32cb + 8(2gp + g2)
        float2 cs[2][2];  // [g2][pair within the 4 channels], shared by both head blocks
        const bool rot = R > 0 && 128 * kq + cb * 32 + 16 * gp >= AD - R;
        if (rot) {
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2)
              cs[g2][i2] = tr[((128 * kq + cb * 32 + 8 * (2 * gp + g2) - (AD - R)) >> 1) + i2];
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          unsigned w[2][2];
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            const int gq = 2 * gp + g2;
            float v[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) v[jj] = o[cb][hb][gq * 4 + jj] * inv[hb];
            if (rot) {
#pragma unroll
              for (int i2 = 0; i2 < 2; ++i2) {
                const float c = cs[g2][i2].x, sn = -cs[g2][i2].y;
                const float xv = v[2 * i2], yv = v[2 * i2 + 1];
                v[2 * i2] = xv * c - yv * sn;
                v[2 * i2 + 1] = xv * sn + yv * c;
              }
            }
            w[g2][0] = pack_bf16x2(v[0], v[1]);
            w[g2][1] = pack_bf16x2(v[2], v[3]);
          }
          // lanes < 32 collect group 2gp (channels +0..7), lanes >= 32 group 2gp+1
          const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
          u32x4_t val;
          val[0] = s0[0];
          val[1] = s1[0];
          val[2] = s0[1];
          val[3] = s1[1];
          // lanes >= 32 write group 2gp + 1: their half * 8 channels are part of ob.  The whole
          // offset goes in the lane offset (a constant SGPR offset on these stores gave
          // corrupted output).
          __builtin_amdgcn_raw_buffer_store_b128(
              val, o_rs, static_cast<unsigned>(ob + (32 * hb * AD + cb * 32 + 2 * gp * 8) * 2), 0, 0);
          __builtin_amdgcn_sched_barrier(0);  // one group at a time: keeps the epilogue's registers few
        }
      }
    }
  };

  // split mode: the unnormalised output of this key range, counter-rotated (the rotation is
  // linear, so it commutes with the merge), as fp32 rows of the workspace
  auto finish_part = [&](int j, int item) {
    const int ln = lane_now();  // offsets formed here, as in finish
    const rsrc_t p_rs = make_rs(a.part + static_cast<size_t>(item) * AH * AD, AH * AD * 4);
    const int ob = ((ln & 31) * AD + 128 * kq + (ln >> 5) * 4) * 4;  // head block 0, channel 128kq
    const float2* tr = reinterpret_cast<const float2*>(lds + RT_OFF + (j & 7) * 256 + (ln >> 5) * 16);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float v[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v[jj] = o[cb][hb][gq * 4 + jj];
          const int cl0 = 128 * kq + cb * 32 + gq * 8;
          if (R > 0 && cl0 >= AD - R) {
            const int pr0 = (cl0 - (AD - R)) >> 1;
#pragma unroll
            for (int i2 = 0; i2 < 4; i2 += 2) {
              const float2 cs = tr[pr0 + i2 / 2];
              const float c = cs.x, sn = -cs.y;
              const float xv = v[i2], yv = v[i2 + 1];
              v[i2] = xv * c - yv * sn;
              v[i2 + 1] = xv * sn + yv * c;
            }
          }
          const u32x4_t val = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                               __float_as_uint(v[3])};
          __builtin_amdgcn_raw_buffer_store_b128(
              val, p_rs, static_cast<unsigned>(ob + (32 * hb * AD + cb * 32 + gq * 8) * 4), 0, 0);
        }
      }
    }
  };

  for (int s = -1;; ++s) {
    lds_barrier();  // X(s): P(s) and the rescale factor are published
    if (s < 0) continue;
    if (jp >= n_mine) break;  // this step would accumulate tile s
    const unsigned char* tb = lds + (s % NSLOT) * ATILE;
    if (tp == 0) {
      if constexpr (CSA) set_keys(cp, __builtin_amdgcn_readfirstlane(nk[jp & 7]), a.n_split);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[cb][hb][e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < VPF; ++i) vr[i] = vfrag(tb, i);
    const int par = s & 1;
    // P^T fragments (ks, hb): head 32hb + l32, keys 16ks + 4half + 0..3 and + 8 (stored
    // contiguously at 16ks + 8half, see the score waves)
    const unsigned char* pt = lds + P_OFF + par * (AH * PPITCH) + l32 * PPITCH + 16 * half;
    bf16x8_t pb[2];  // the current key half's fragments, one per head block
    auto pfrag = [&](int ks) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        pb[hb] = *reinterpret_cast<const bf16x8_t*>(pt + hb * (32 * PPITCH) + 32 * ks);
    };
    pfrag(0);
    float alpha[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) alpha[hb] = alph[par * 64 + 32 * hb + l32];
    if (__ballot(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[cb][hb][e] *= alpha[hb];
    }
#pragma unroll
    for (int st = 0; st < 2 * NCB; ++st) {
      if (st == NCB) pfrag(1);  // the first half's fragments are done
      const bf16x8_t vf = vr[st % VPF];
      if (st + VPF < 2 * NCB) vr[st % VPF] = vfrag(tb, st + VPF);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        o[st % NCB][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[hb], o[st % NCB][hb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (tp + 1 == cp.n_tiles) {
      if (a.n_split > 1) {
        finish_part(jp, qid_of(jp));
      } else {
        const int l = lane_now() & 31;
        const float inv[2] = {1.f / lsum[par * 64 + l], 1.f / lsum[par * 64 + 32 + l]};
        finish(cp, jp, inv);
      }
      tp = 0;
      if (++jp < n_mine) cp = query_geom<CSA>(a, qid_of(jp));
      else break;  // that was the last tile: step n_tiles - 1 is done
    } else {
      ++tp;
    }
  }
}

// Split-mode merge: per (query, head, 4 channels), the partial outputs of the key ranges are
// combined in the common scale of their largest running max.  Every range started from the
// sink state (max = sink, sum = 1), so n_split - 1 copies of the sink term are removed.
// NS ranges, a compile-time count: every range's (max, sum) pair and partial output is
// loaded before any is used (in a loop over a run-time count each load was waited for in
// turn).
template <int NS>
__global__ void __launch_bounds__(256) attend_merge_kernel(const float* __restrict__ part,
                                                           const float* __restrict__ sink,
                                                           bf16_t* __restrict__ out, int n_q) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid >= n_q * AH * (AD / 4)) return;
  const int q = gid / (AH * (AD / 4));
  const int h = (gid / (AD / 4)) % AH;
  const int c = (gid % (AD / 4)) * 4;
  const float* ml = part + static_cast<size_t>(n_q) * NS * AH * AD;
  float2 mls[NS];
  f32x4_t v[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const size_t item = static_cast<size_t>(q) * NS + i;
    mls[i] = *reinterpret_cast<const float2*>(ml + (item * AH + h) * 2);
    v[i] = *reinterpret_cast<const f32x4_t*>(part + (item * AH + h) * AD + c);
  }
  const float sink2 = sink[h] * kLog2e;
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NS; ++i) mx = fmaxf(mx, mls[i].x);
  float l = -static_cast<float>(NS - 1) * __builtin_amdgcn_exp2f(sink2 - mx);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const float w = __builtin_amdgcn_exp2f(mls[i].x - mx);
    l += w * mls[i].y;
    acc += w * v[i];
  }
  const float inv = 1.f / l;
  u32x2_t pk;
  pk[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2_t*>(out + (static_cast<size_t>(q) * AH + h) * AD + c) = pk;
}

static int device_cus() {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      n_cu = n > 0 ? n : 1;
    else
      return 1;
  }
  return n_cu;
}

constexpr int kMaxSplit = 8;

int attend_split_count(int n_q) {
  if (n_q <= 0) return 1;
  const int n = device_cus() / n_q;
  return n < 2 ? 1 : (n > kMaxSplit ? kMaxSplit : n);
}

size_t attend_split_bytes(int n_q) {
  const int ns = attend_split_count(n_q);
  if (ns < 2) return 0;
  return static_cast<size_t>(n_q) * ns * (AH * AD + AH * 2) * sizeof(float);
}

bool attend_fast(int H, int D, int r, int dtype) {
  return dtype == 1 && H == AH && D == AD && (r == 0 || r == 64);
}

bool attend_uses_fast(const AttendArgs& a) {
  // a batch's window / pool slice must be addressable with 32-bit buffer offsets
  constexpr long long kMaxRows = (1LL << 22) - 8;
  return attend_fast(a.H, a.D, a.r, a.dtype) && (!a.csa || a.k <= kMaxTopk) && a.S_kv <= kMaxRows &&
         a.N_cap <= kMaxRows;
}

hipError_t launch_attend_generic(const AttendArgs& a, hipStream_t st);

template <bool CSA, int R>
static hipError_t launch_mfma(const AttendArgs& a, hipStream_t st) {
  static bool attr_set = false;  // per instantiation; setting it again is harmless
  static int n_cu = 0;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_mfma_kernel<CSA, R>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n_cu < 1) n_cu = 1;
    attr_set = true;
  }
  const int n_q = a.B * a.T;
  const int n_items = n_q * a.n_split;
  const unsigned blocks = static_cast<unsigned>(n_items < n_cu ? n_items : n_cu);
  hipLaunchKernelGGL((attend_mfma_kernel<CSA, R>), dim3(blocks), dim3(640), kLdsBytes, st, a);
  if (a.n_split > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int total = n_q * AH * (AD / 4);
    const dim3 grid((total + 255) / 256);
    bf16_t* out = static_cast<bf16_t*>(a.out);
    switch (a.n_split) {
#define MERGE(ns) \
  case ns: hipLaunchKernelGGL(attend_merge_kernel<ns>, grid, dim3(256), 0, st, a.part, a.sink, out, n_q); break;
      MERGE(2) MERGE(3) MERGE(4) MERGE(5) MERGE(6) MERGE(7) MERGE(8)
#undef MERGE
      default: return hipErrorInvalidValue;  // attend_split_count gives 1 .. kMaxSplit
    }
  }
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  if (a.pairs) return launch_attend_dense(a, st);  // shape checked by the caller
  if (attend_uses_fast(a)) {
    if (a.r == 64) return a.csa ? launch_mfma<true, 64>(a, st) : launch_mfma<false, 64>(a, st);
    return a.csa ? launch_mfma<true, 0>(a, st) : launch_mfma<false, 0>(a, st);
  }
  return launch_attend_generic(a, st);
}

}  // namespace dsv4
