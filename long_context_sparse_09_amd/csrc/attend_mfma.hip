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
//   * Persistent workgroups (one per CU) walk their queries as one stream of 32-key tiles.
//     While a query's last tile computes, the next query's first tile is already being
//     gathered and its Q rows are loading, so per-query set-up overlaps compute.
//   * Query order: heaviest first, and each round hands G/8 consecutive queries to the G/8
//     workgroups of one XCD, so the window rows that neighbouring queries share are fetched
//     into that XCD's L2 once.  Q is loaded and the output stored non-temporally, keeping the
//     pool and window rows resident in L2.
//   * 4 wavefronts; wave (hb, kh) owns heads [32hb, 32hb+32) and channels [256kh, 256kh+256).
//   * Gather: a tile's 32 key rows (window rows, then the selected / visible pool rows) go
//     straight from global memory into LDS (global_load_lds, one 1 KB row per wave
//     instruction), double-buffered.  Row addresses come from one vector op, read out per row
//     with readlane.
//   * QK^T is split over channels: wave (hb, kh) forms the partial S^T = K[:, ch kh] .
//     Q^T[ch kh] (v_mfma_f32_32x32x16_bf16; A = 32 key rows from LDS, B = its half of the
//     rotated Q, kept in registers), the two waves of a head block swap partials through LDS,
//     and both then hold the same full logits (each lane: 16 keys of ONE head).  They run the
//     same online softmax, so no further exchange is needed.
//   * The S^T accumulator layout is exactly the B operand of O^T = V^T . P^T, so P goes from
//     accumulator to operand in registers; V^T (A operand) comes from the same row-major tile
//     through ds_read_tr16_b64 (transposing 4 x 16 LDS reads): K = V is stored once.
//   * The running max is moved only when a logit exceeds it by 2^8 (lazy rescale).  The state
//     starts from the sink: max = s_h, sum = 1, value 0.
//   * LDS rows are 1024 B with their 16-byte chunks XOR-swizzled per row (chunk c of row r
//     sits at c ^ f(r), f(r) = 2(r mod 4) + ((r >> 2) mod 2)), so the 8-row b128 reads of QK^T
//     and the 4-row transposing reads of PV each touch distinct banks.
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

constexpr int AH = 64;                   // query heads
constexpr int AD = 512;                  // head_dim
constexpr int ANK = 32;                  // keys per tile
constexpr int APITCH = AD * 2;           // LDS bytes per key row (swizzled, no pad)
constexpr int ATILE = ANK * APITCH;      // bytes per tile buffer
constexpr int ATILES_BYTES = 2 * ATILE;  // double buffer
constexpr int AXS_BYTES = 2 * 4 * 16 * 64 * 4;  // partial-logit exchange: [parity][hb,kh][16][64]
constexpr float kLazy = 8.f;             // log2-domain headroom before the running max moves
constexpr int kMaxTopk = 1024;           // key-list capacity per buffer on this path
constexpr int kMaxDynLds = ATILES_BYTES + AXS_BYTES + 2 * kMaxTopk * 4;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

__device__ __forceinline__ int swz(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }

// Per-query description, identical in every thread of the workgroup.
struct QDesc {
  int b, t, r0, n_win, n_keys, n_tiles, buf;
  long long p;
};

}  // namespace

template <bool CSA, int R>  // R = rotary channels, 0 or 64 (compile-time: only those chunks move)
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
attend_mfma_kernel(AttendArgs a) {
  static_assert(R == 0 || R == 64, "rotary width on this path");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* tiles = lds;
  f32x4_t* xs = reinterpret_cast<f32x4_t*>(lds + ATILES_BYTES);           // [2][4][4][64]
  int* klist = reinterpret_cast<int*>(lds + ATILES_BYTES + AXS_BYTES);    // CSA: [2][k]
  __shared__ float rope_c[2][kMaxRope / 2], rope_s[2][kMaxRope / 2];
  __shared__ int wave_tot[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int hb = wave & 1, kh = wave >> 1;
  const int head = hb * 32 + l32;
  const int n_q = a.B * a.T;
  const int G = gridDim.x;
  const float c2 = a.scale * kLog2e;  // logits in the log2 domain
  const float sink2 = a.sink[head] * kLog2e;
  const bf16_t* qbase = static_cast<const bf16_t*>(a.q);

  // j-th query of this workgroup, as a rank in the heaviest-first order.  Workgroups are
  // dealt to the 8 XCDs round-robin; with G a multiple of 8, round j gives XCD x the ranks
  // [jG + xG/8, jG + (x+1)G/8), i.e. G/8 consecutive queries.
  const int g = static_cast<int>(blockIdx.x);
  const int slot = (G % 8) == 0 ? (g % 8) * (G / 8) + g / 8 : g;
  const int n_mine = (n_q - slot + G - 1) / G;

  // ---- per-query set-up: position, window rows, key list, rope table (all threads) ----
  auto prepare = [&](int j, QDesc& d, int buf) {
    const int qid = n_q - 1 - (j * G + slot);
    d.b = qid / a.T;
    d.t = qid % a.T;
    d.buf = buf;
    d.p = static_cast<long long>(a.q_pos0[d.b]) + d.t;
    const long long lo = max(0LL, d.p - a.window + 1);
    d.r0 = static_cast<int>(max(lo - a.kv_pos0[d.b], 0LL));
    const int r1 = static_cast<int>(min(d.p + 1 - a.kv_pos0[d.b], static_cast<long long>(a.S_kv)));
    d.n_win = max(0, r1 - d.r0);
    __syncthreads();  // earlier readers of klist[buf] / rope[buf] are done
    if (tid < R / 2) {  // one (cos, sin) per rotary pair: angle in double, reduced mod 2pi
      const double turns = static_cast<double>(d.p + a.pos_off) * a.inv_freq[tid] *
                           0.15915494309189533576888376337251;  // 1 / (2 pi)
      const float frac = static_cast<float>(turns - rint(turns));  // in [-1/2, 1/2]
      rope_c[buf][tid] = __builtin_amdgcn_cosf(frac);  // hardware sin/cos take turns
      rope_s[buf][tid] = __builtin_amdgcn_sinf(frac);
    }
    int n_cmp;
    if constexpr (CSA) {
      const int* idx = a.topk_idx + (static_cast<size_t>(d.b) * a.T + d.t) * a.k;
      int* kl = klist + buf * a.k;
      int base = 0;
      for (int c0 = 0; c0 < a.k; c0 += 256) {
        const int i = c0 + tid;
        const int e = i < a.k ? idx[i] : -1;
        const bool v = e >= 0 && e < a.N_cap;
        int tot;
        const int pos = base + block_excl_count<256>(v, &tot, wave_tot);
        if (v) kl[pos] = e;
        base += tot;
      }
      n_cmp = base;
    } else {
      long long v = a.N_cap > 0 ? (d.p + 1) / a.m_hca : 0;
      v = min(v, static_cast<long long>(a.n_pool ? a.n_pool[d.b] : a.N_cap));
      v = min(v, static_cast<long long>(a.N_cap));
      n_cmp = static_cast<int>(max(v, 0LL));
    }
    d.n_keys = d.n_win + n_cmp;
    d.n_tiles = max(1, (d.n_keys + ANK - 1) / ANK);  // an empty query still runs one masked tile
    __syncthreads();
  };

  const bf16_t* win0 = static_cast<const bf16_t*>(a.kv_win);
  const bf16_t* pool0 = static_cast<const bf16_t*>(a.pool);
  // Gather of tile `it` of query d into tile buffer `tbuf`, in two steps: tile_addr() forms,
  // in lane l < 32, the address of key it*32 + l; issue_row(p) then moves row p*4 + wave
  // (1 KB, read out with readlane) straight into LDS, every lane fetching the logical chunk
  // that belongs at its physical (swizzled) LDS position.  The 8 row moves of a wave are
  // interleaved with the QK^T MFMAs so that issue stalls overlap matrix work.
  unsigned rlo = 0, rhi = 0;
  unsigned char* gtb = tiles;
  auto tile_addr = [&](const QDesc& d, int it, int tbuf) {
    const int x = it * ANK + l32;
    const bf16_t* row;
    if (x < d.n_keys) {
      if (x < d.n_win) {
        row = win0 + (static_cast<size_t>(d.b) * a.S_kv + d.r0 + x) * AD;
      } else {
        const int e = CSA ? klist[d.buf * a.k + x - d.n_win] : x - d.n_win;
        row = pool0 + (static_cast<size_t>(d.b) * a.N_cap + e) * AD;
      }
    } else {  // masked filler: the query's own first row (in bounds, finite)
      row = qbase + (static_cast<size_t>(d.b) * a.T + d.t) * AH * AD;
    }
    const unsigned long long rp = reinterpret_cast<unsigned long long>(row);
    rlo = static_cast<unsigned>(rp);
    rhi = static_cast<unsigned>(rp >> 32);
    gtb = tiles + tbuf * ATILE;
  };
  auto issue_row = [&](int pass) {
    const int r = pass * 4 + wave;
    const unsigned lo32 = __builtin_amdgcn_readlane(rlo, r);
    const unsigned hi32 = __builtin_amdgcn_readlane(rhi, r);
    const unsigned char* src = reinterpret_cast<const unsigned char*>(
        (static_cast<unsigned long long>(hi32) << 32) | lo32);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + ((lane ^ swz(r)) << 4)),
                                     (lds_void*)(gtb + r * APITCH), 16, 0, 0);
  };
  auto issue_tile = [&](const QDesc& d, int it, int tbuf) {
    tile_addr(d, it, tbuf);
#pragma unroll
    for (int pass = 0; pass < ANK / 4; ++pass) issue_row(pass);
  };

  // This wave's half of Q^T (B operand): head hb*32 + l32, channels kh*256 + ks*16 + half*8
  constexpr int NKS = AD / 2 / 16;
  bf16x8_t qf[NKS];
  auto load_q = [&](const QDesc& d) {
    const bf16_t* qrow = qbase + ((static_cast<size_t>(d.b) * a.T + d.t) * AH + head) * AD +
                         kh * (AD / 2) + half * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = __builtin_bit_cast(
          bf16x8_t, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(qrow + ks * 16)));
  };
  // rotary channels 448..511 = the last R/16 chunks of the kh = 1 half
  auto rotate_q = [&](const QDesc& d) {
    if (R == 0 || kh == 0) return;
#pragma unroll
    for (int ks = NKS - R / 16; ks < NKS; ++ks) {
      const int pr0 = (ks * 16 + half * 8 - (AD / 2 - R)) >> 1;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float c = rope_c[d.buf][pr0 + i / 2], sn = rope_s[d.buf][pr0 + i / 2];
        const float xv = static_cast<float>(qf[ks][i]), yv = static_cast<float>(qf[ks][i + 1]);
        qf[ks][i] = static_cast<__bf16>(xv * c - yv * sn);
        qf[ks][i + 1] = static_cast<__bf16>(xv * sn + yv * c);
      }
    }
  };

  // lane-constant LDS offsets of the swizzled layout
  int qk_off[4];  // QK^T A operand: row l32, chunk kh*32 + 2*(ks%4) + half (+ 8*(ks/4))
  {
    const int f = swz(l32);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      qk_off[jj] = l32 * APITCH + kh * 4 * 128 + (((2 * jj + half) ^ f) << 4);
  }
  // PV transposing reads: rows 16ss + 4*half + n16/4 (+8), channels kh*256 + dt*32 + dh*16
  // + 4*(n16%4); the 16-byte chunk of that column is XOR-ed with f = swz(row) = 2(n16/4)+half
  int tr_off[2];
  {
    const int n16 = lane & 15, dh = (lane >> 4) & 1;
    const int f = 2 * (n16 >> 2) + half;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      tr_off[jj] = (4 * half + (n16 >> 2)) * APITCH + kh * 4 * 128 +
                   (((4 * jj + 2 * dh + ((n16 & 3) >> 1)) ^ f) << 4) + (n16 & 1) * 8;
  }

  constexpr int NDT = AD / 2 / 32;  // output channel tiles owned by this wave
  f32x16_t o[NDT];
  float m_run = sink2, l_run = 1.f;
  auto reset = [&]() {
    m_run = sink2;
    l_run = 1.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  };

  // ---- epilogue of one query: normalise, counter-rotate (eq. 26), store ----
  // The finished tile buffer (32 KB, free once the workgroup has synchronised) stages the
  // output so that stores are contiguous: in round hr, wave (hb, kh) writes channels
  // kh*256 + [128hr, 128hr+128) of its 32 heads (8 KB: row = head, 16 chunks of 16 B, chunk c
  // of row h at c ^ (h mod 16)) into its quarter, then each store instruction writes 4 heads x
  // 256 contiguous bytes.
  auto finish = [&](const QDesc& d, unsigned char* stage) {
    const float inv = 1.f / l_run;
    unsigned char* wst = stage + wave * 8192;
    bf16_t* obase = static_cast<bf16_t*>(a.out) +
                    ((static_cast<size_t>(d.b) * a.T + d.t) * AH + hb * 32) * AD + kh * (AD / 2);
#pragma unroll
    for (int hr = 0; hr < 2; ++hr) {
#pragma unroll
      for (int dq = 0; dq < NDT / 2; ++dq) {
        const int dt = hr * (NDT / 2) + dq;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float v[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v[jj] = o[dt][gq * 4 + jj] * inv;
          const int cl = dt * 32 + gq * 8 + half * 4;  // channel within this wave's half
          if (R > 0 && kh == 1 && cl >= AD / 2 - R) {  // the same angle, negated
            const int pr0 = (cl - (AD / 2 - R)) >> 1;
#pragma unroll
            for (int i2 = 0; i2 < 4; i2 += 2) {
              const float c = rope_c[d.buf][pr0 + i2 / 2], sn = rope_s[d.buf][pr0 + i2 / 2];
              const float xv = v[i2], yv = v[i2 + 1];
              v[i2] = xv * c + yv * sn;
              v[i2 + 1] = -xv * sn + yv * c;
            }
          }
          u32x2_t pk2;
          pk2[0] = pack_bf16x2(v[0], v[1]);
          pk2[1] = pack_bf16x2(v[2], v[3]);
          const int chunk = (dq * 4 + gq) ^ (l32 & 15);  // head l32, channels (dq*4+gq)*8 ..
          *reinterpret_cast<u32x2_t*>(wst + l32 * 256 + chunk * 16 + half * 8) = pk2;
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2) {  // lane l: head 4*k2 + l/16, 16-byte chunk l%16
        const int hh = 4 * k2 + (lane >> 4), ch = lane & 15;
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(wst + hh * 256 + ((ch ^ (hh & 15)) << 4));
        __builtin_nontemporal_store(
            val, reinterpret_cast<u32x4_t*>(obase + static_cast<size_t>(hh) * AD + hr * 128 + ch * 8));
      }
    }
  };

  QDesc cur, nxt;
  prepare(0, cur, 0);
  load_q(cur);
  issue_tile(cur, 0, 0);
  int j = 0, it = 0, tbuf = 0, par = 0;

  for (;;) {
    if (it == 0) {  // a new query starts: set up the following one, then this one's Q and state
      if (j + 1 < n_mine) prepare(j + 1, nxt, cur.buf ^ 1);
      rotate_q(cur);
      reset();
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's gather of the current tile has landed
    __syncthreads();                // ... and every wave's; the other tile buffer is free
    const bool last = (it + 1 == cur.n_tiles);
    const bool more = (j + 1 < n_mine);
    const bool fetch = !last || more;
    if (fetch) tile_addr(last ? nxt : cur, last ? 0 : it + 1, tbuf ^ 1);
    const unsigned char* tb = tiles + tbuf * ATILE;

    // partial S^T (32 keys x 32 heads) over this wave's 256 channels; K fragments run 4 ahead,
    // one gather row move after every second MFMA
    f32x16_t s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    {
      constexpr int PF = 4;
      bf16x8_t kr[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) kr[i] = *reinterpret_cast<const bf16x8_t*>(tb + qk_off[i]);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8_t kf = kr[ks % PF];
        if (ks + PF < NKS)
          kr[ks % PF] = *reinterpret_cast<const bf16x8_t*>(tb + qk_off[(ks + PF) & 3] + ((ks + PF) >> 2) * 128);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
        if ((ks & 1) && fetch) issue_row(ks >> 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (last && more) load_q(nxt);  // the next query's Q streams in behind this tile

    // swap partial logits with the other channel half of this head block
    f32x4_t* xme = xs + ((par * 4 + hb * 2 + kh) * 4) * 64 + lane;
    const f32x4_t* xpa = xs + ((par * 4 + hb * 2 + (kh ^ 1)) * 4) * 64 + lane;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) xme[q4 * 64] = f32x4_t{s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
    __syncthreads();
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4_t pv4 = xpa[q4 * 64];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * q4 + i] += pv4[i];
    }

    // online softmax over the tile's 32 keys (lane: head l32, keys (e/4)*8 + half*4 + e%4);
    // both waves of the head block compute the same values
    const int kbase = it * ANK + half * 4;
    float tmax = -INFINITY;
    if (it * ANK + ANK > cur.n_keys) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + (e >> 2) * 8 + (e & 3);
        s[e] = key < cur.n_keys ? s[e] * c2 : -INFINITY;
        tmax = fmaxf(tmax, s[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] *= c2;
        tmax = fmaxf(tmax, s[e]);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = (tmax > m_run + kLazy) ? tmax : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8_t pb[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = __builtin_amdgcn_exp2f(s[e] - m_new);
      psum += pv;
      pb[e >> 3][e & 7] = static_cast<__bf16>(pv);
    }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    if (__ballot(m_new != m_run)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
    }
    m_run = m_new;

    // O^T (32 channels x 32 heads per tile dt) += V^T (32 channels x 16 key slots) . P^T
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      const unsigned char* vb = tb + 16 * ss * APITCH;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const unsigned char* va = vb + tr_off[dt & 1] + (dt >> 1) * 128;
        const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(va));
        const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(va + 8 * APITCH));
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[ss], o[dt], 0, 0, 0);
      }
    }

    if (last) {
      __syncthreads();  // every wave is done with this tile buffer: it stages the output
      finish(cur, tiles + tbuf * ATILE);
    }
    par ^= 1;
    tbuf ^= 1;
    if (!last) {
      ++it;
      continue;
    }
    if (!more) break;
    cur = nxt;
    ++j;
    it = 0;
  }
}

bool attend_fast(int H, int D, int r, int dtype) {
  return dtype == 1 && H == AH && D == AD && (r == 0 || r == 64);
}

bool attend_uses_fast(const AttendArgs& a) {
  return attend_fast(a.H, a.D, a.r, a.dtype) && (!a.csa || a.k <= kMaxTopk);
}

hipError_t launch_attend_generic(const AttendArgs& a, hipStream_t st);

template <bool CSA, int R>
static hipError_t launch_mfma(const AttendArgs& a, hipStream_t st) {
  const size_t shmem =
      ATILES_BYTES + AXS_BYTES + (CSA ? 2 * static_cast<size_t>(a.k) * sizeof(int) : 0);
  static bool attr_set = false;  // per instantiation; setting it again is harmless
  static int n_cu = 0;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_mfma_kernel<CSA, R>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDynLds);
    if (e != hipSuccess) return e;
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n_cu < 1) n_cu = 1;
    attr_set = true;
  }
  const int n_q = a.B * a.T;
  const unsigned blocks = static_cast<unsigned>(n_q < n_cu ? n_q : n_cu);
  hipLaunchKernelGGL((attend_mfma_kernel<CSA, R>), dim3(blocks), dim3(256), shmem, st, a);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  if (attend_uses_fast(a)) {
    if (a.r == 64) return a.csa ? launch_mfma<true, 64>(a, st) : launch_mfma<false, 64>(a, st);
    return a.csa ? launch_mfma<true, 0>(a, st) : launch_mfma<false, 0>(a, st);
  }
  return launch_attend_generic(a, st);
}

}  // namespace dsv4
