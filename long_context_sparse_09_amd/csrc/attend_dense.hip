// Dense-range attention on MFMA for gfx950 (bf16 storage, fp32 accumulation), 64 query heads x
// head_dim 512, for the layers whose keys are a contiguous range: HCA (the window rows, then
// every visible pool entry) and sliding-window layers (the window rows only).
//
// Source: DeepSeek-V4 model page (Transformers docs), "Hybrid attention (§2.3)": HCA attends to
// every pool entry (no indexer), one K=V head read as both key and value, partial RoPE on the
// trailing channels, the output rope slice rotated at position -i (eq. 26), a per-head sink
// (eq. 27), the sliding-window branch before the compressed keys.  "Attention mask layout",
// HCA paragraph: entry w is visible to query t iff w < (t+1) // m'; the window keeps the last
// sliding_window tokens up to the query.
//
// Two consecutive queries of a sequence see almost the same keys: their windows share all but
// one row at each end, and their visible pool entries are the same except when a pool entry
// closes between them.  One workgroup therefore takes a PAIR of queries and streams the union
// of their keys (window rows of the earlier query's first row .. the later query's own row,
// then the later query's visible entries) once, in 32-key tiles; each key tile is read from
// LDS by 128 query-head rows (2 queries x 64 heads) instead of 64.
//
//   * Four wavefronts, one per SIMD, each owning 32 rows: wave w takes query w >> 1 of the
//     pair, heads 32 (w & 1) .. +31, over all 512 channels.  Nothing passes between waves but
//     the key tiles: QK^T (S^T = K . Q^T, 32 x 32 x 16 bf16 MFMA, 32 per tile), the online
//     softmax and PV (O^T = V^T . P^T, 32 per tile) all run in the wave that owns the rows.
//     Q (32 heads x 512, bf16) stays in registers, the output (32 heads x 512, fp32) in
//     accumulator registers; 1 wave per SIMD holds both.
//   * The S^T accumulator already has the B-operand layout PV needs (lane: one head, 8 of the
//     16 keys of a half), with key bits 2 and 3 swapped within each 16-key block; the V^T
//     fragments are read in that key order by transposing LDS reads (ds_read_tr16_b64).
//   * Key tiles move from global memory straight into LDS (buffer_load ... lds), each wave
//     one quarter of the rows, into a ring of four 32 KB tiles filled three tiles ahead; one
//     workgroup barrier per tile.  Rows keep their 16-byte chunks XOR-swizzled (chunk c of
//     row r at c ^ (4(r mod 4) + (r/4 mod 4))), so both read patterns are conflict-free.
//   * Online softmax in the log2 domain, state seeded from the sink (max = s_h, sum = 1); the
//     running max moves only when a logit exceeds it by 2^8 (lazy rescale), so the output
//     accumulators are rescaled rarely.
//   * Keys a row must not see (the other query's end rows, entries that close between the two
//     queries, the ragged last tile) are masked per key on the tiles that hold them.
//   * Persistent workgroups, pairs heaviest first, consecutive pairs on one XCD (they share
//     window rows in its L2).
//
// This kernel serves hca_attend_pairs.  hca_attend keeps the per-query kernel: with one wave
// per SIMD every wave issues its share of the key-row copies, a wave stalls ~200 cycles per
// 1 KB copy it issues, and nothing else keeps its SIMD's matrix core busy meanwhile, while the
// per-query kernel gives the copies to waves of their own (HCA S=65536: 5.7 ms here, 4.6 ms
// per query).
#include "common.h"
#include "launch.h"

namespace dsv4 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 dbf16x8_t;
typedef __attribute__((ext_vector_type(4))) short di16x4_t;
typedef __attribute__((ext_vector_type(16))) float df32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned du32x4_t;
typedef __attribute__((address_space(3))) void dlds_void;
typedef __attribute__((address_space(3))) di16x4_t dlds_i16x4;
typedef __amdgpu_buffer_rsrc_t drsrc_t;

constexpr int QH = 64;               // query heads
constexpr int QD = 512;              // head_dim
constexpr int TK = 32;               // keys per tile
constexpr int ROWB = QD * 2;         // LDS bytes per key row
constexpr int TILEB = TK * ROWB;     // bytes per tile buffer
constexpr int NRING = 4;             // tile ring
constexpr int RT_OFF = NRING * TILEB;  // per-wave RoPE (cos, sin) table: [wave][32 pairs]
constexpr int kDenseLds = RT_OFF + 4 * 32 * 8;
static_assert(kDenseLds <= 160 * 1024, "LDS budget");
constexpr float kLazyMax = 8.f;
constexpr double kTurn = 0.15915494309189533576888376337251;  // 1 / (2 pi)
constexpr int kWord3 = 0x00020000;   // raw buffer

__device__ __forceinline__ int dswz(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }

__device__ __forceinline__ drsrc_t rs_of(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           kWord3);
}

__device__ __forceinline__ int uload(const int* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) int*>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ float swap_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS-only workgroup barrier: drains this wave's LDS operations, not its vector-memory ones
// (the tile loads in flight are waited for explicitly).
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// vmcnt(n) for the counts this kernel needs (n < 64): the immediate keeps lgkmcnt and expcnt open.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// o += a . b on v_mfma_f32_32x32x16_bf16 with the accumulator pinned to accumulator
// registers: the output (256 per lane) fills them, and left to itself the register allocator
// moved output blocks between register files around every instruction.  Written as inline
// asm, so its hazards are covered by hand: its operands are produced at least 5 wait states
// ahead (s_nop before the first), an accumulator is never the next instruction's, and every
// VALU access of the output waits for the last instruction (drain_pv).
__device__ __forceinline__ void pv_mfma(df32x16_t& o, const dbf16x8_t& a, const dbf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}
// Output accumulators are only touched through these (and pv_mfma), so that the register
// allocator keeps them in accumulator registers.
__device__ __forceinline__ float acc_read(const float& x) {
  float t;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(x));
  return t;
}
__device__ __forceinline__ void zero_acc(df32x16_t& o) {
#pragma unroll
  for (int e = 0; e < 16; ++e) asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(o[e]));
}
// o *= f in place, one accumulator register at a time (written as plain vector code, the
// whole output was copied to vector registers and spilled)
__device__ __forceinline__ void scale_acc(df32x16_t& o, float f) {
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float t;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(o[e]));
    t *= f;
    asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(o[e]) : "v"(t));
  }
}
__device__ __forceinline__ void drain_mfma() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
// s += a . b (s in vector registers: the accumulator registers all hold the output); the
// first of a chain starts from zero.  Consecutive instructions of the chain accumulate into
// the same registers (the dependent-accumulation case the matrix core forwards).
__device__ __forceinline__ void qk_mfma_first(df32x16_t& s, const dbf16x8_t& a, const dbf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(a), "v"(b));
}
__device__ __forceinline__ void qk_mfma(df32x16_t& s, const dbf16x8_t& a, const dbf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "v"(b));
}

// One 1 KB key row from global memory into LDS (buffer_load ... lds, 16 bytes per lane).
// Issued as inline asm: after the builtin form, the compiler put a wait for every vector-memory
// operation before the next LDS reads (it cannot tell that the copy does not touch what they
// read), which drained the tiles in flight every step.  Every consumer of the tiles waits for
// them explicitly (vmcnt + workgroup barrier).  The descriptor and M0 are written by scalar
// code (M0 set by the compiler from the asm's input operand); five wait states precede the
// load.
typedef __attribute__((ext_vector_type(4))) unsigned dsu32x4_t;
__device__ __forceinline__ void dma_row(const void* src, unsigned char* dst, unsigned voff) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(src);
  dsu32x4_t rs;
  rs[0] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(p));
  rs[1] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(p >> 32)) & 0xFFFFu;
  rs[2] = ROWB;
  rs[3] = kWord3;
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<uintptr_t>((dlds_void*)dst)));
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "{m0}"(m0)
               : "memory");
}

// One work item: a pair of consecutive queries t0, t0 + 1 of sequence b (or t0 alone at the
// end of an odd-length sequence).  Key g of the pair's stream is window row wr0 + g for
// g < n_win, pool entry g - n_win for n_win <= g < n_keys.
struct Pair {
  int b, t0, two, wr0, n_win, n_keys, n_tiles;
  long long p0;
};

__device__ __forceinline__ int pool_visible(const AttendArgs& a, int b, long long p) {
  if (a.N_cap <= 0) return 0;
  long long v = (p + 1) / a.m_hca;
  v = min(v, static_cast<long long>(a.n_pool ? uload(a.n_pool + b) : a.N_cap));
  v = min(v, static_cast<long long>(a.N_cap));
  return static_cast<int>(max(v, 0LL));
}

__device__ __forceinline__ Pair pair_of(const AttendArgs& a, int item, int per_seq) {
  Pair d;
  d.b = item / per_seq;
  d.t0 = 2 * (item - d.b * per_seq);
  d.two = d.t0 + 1 < a.T ? 1 : 0;
  d.p0 = static_cast<long long>(uload(a.q_pos0 + d.b)) + d.t0;
  const long long p_last = d.p0 + d.two;
  const int kv0 = uload(a.kv_pos0 + d.b);
  const long long lo = max(0LL, d.p0 - a.window + 1);
  d.wr0 = static_cast<int>(max(lo - kv0, 0LL));
  const int r1 = static_cast<int>(min(p_last + 1 - kv0, static_cast<long long>(a.S_kv)));
  d.n_win = max(0, r1 - d.wr0);
  d.n_keys = d.n_win + pool_visible(a, d.b, p_last);
  d.n_tiles = max(1, (d.n_keys + TK - 1) / TK);
  d.b = __builtin_amdgcn_readfirstlane(d.b);
  d.t0 = __builtin_amdgcn_readfirstlane(d.t0);
  d.two = __builtin_amdgcn_readfirstlane(d.two);
  d.wr0 = __builtin_amdgcn_readfirstlane(d.wr0);
  d.n_win = __builtin_amdgcn_readfirstlane(d.n_win);
  d.n_keys = __builtin_amdgcn_readfirstlane(d.n_keys);
  d.n_tiles = __builtin_amdgcn_readfirstlane(d.n_tiles);
  return d;
}

// Keys g the wave's query sees: [glo, ghi) of the window part, [n_win, n_win + vq) of the pool.
struct Seen {
  int glo, ghi, pend;  // pend = n_win + visible entries
  long long p;         // sequence index of the query
  int t;               // query index
};

__device__ __forceinline__ Seen seen_of(const AttendArgs& a, const Pair& d, int qsel) {
  Seen s;
  const int q = d.two ? qsel : 0;  // a lone query: both halves of the workgroup take it
  s.t = d.t0 + q;
  s.p = d.p0 + q;
  const int kv0 = uload(a.kv_pos0 + d.b);
  const long long lo = max(0LL, s.p - a.window + 1);
  const int r0 = static_cast<int>(max(lo - kv0, 0LL));
  const int r1 = static_cast<int>(min(s.p + 1 - kv0, static_cast<long long>(a.S_kv)));
  s.glo = __builtin_amdgcn_readfirstlane(min(max(r0 - d.wr0, 0), d.n_win));
  s.ghi = __builtin_amdgcn_readfirstlane(min(max(r1 - d.wr0, s.glo), d.n_win));
  s.pend = __builtin_amdgcn_readfirstlane(d.n_win + pool_visible(a, d.b, s.p));
  s.t = __builtin_amdgcn_readfirstlane(s.t);
  return s;
}

}  // namespace

template <int R>  // rotary channels: 0 or 64
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attend_dense_kernel(AttendArgs a) {
  static_assert(R == 0 || R == 64, "rotary width on this path");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int qsel = wave >> 1;            // query of the pair
  const int head = 32 * (wave & 1) + l32;  // this lane's head
  const int per_seq = (a.T + 1) / 2;
  const int n_items = a.B * per_seq;
  const int G = gridDim.x;
  const int g = static_cast<int>(blockIdx.x);
  const int slot = (G % 8) == 0 ? (g % 8) * (G / 8) + g / 8 : g;
  const int n_mine = (n_items - slot + G - 1) / G;
  auto item_of = [&](int j) { return n_items - 1 - (j * G + slot); };  // heaviest first

  const bf16_t* qbase = static_cast<const bf16_t*>(a.q);
  const bf16_t* winb = static_cast<const bf16_t*>(a.kv_win);
  const bf16_t* poolb = static_cast<const bf16_t*>(a.pool);
  float2* rtab = reinterpret_cast<float2*>(lds + RT_OFF) + wave * 32;

  // ---------------------------------------------------------------- tile fill
  // Wave w moves rows 8w .. 8w + 7 of each tile.  Lane l writes LDS chunk l of the row with
  // the row's global chunk l ^ swz(row).
  unsigned fvoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) fvoff[i] = static_cast<unsigned>((lane ^ dswz(8 * wave + i)) << 4);
  int fj = 0, ft = 0;  // fill cursor: item rank, tile
  Pair fp = pair_of(a, item_of(0), per_seq);
  int n_issued = 0;
  bool fmore = n_mine > 0;
  // row i (0..7) of this wave's share of the tile at the fill cursor
  auto issue_row = [&](int i) {
    // row sources are wave-uniform: scalar selects, one row descriptor per row
    const int r = 8 * wave + i;
    const int key = ft * TK + r;
    const bf16_t* src;
    if (key < fp.n_win) {
      src = winb + (static_cast<size_t>(fp.b) * a.S_kv + fp.wr0 + key) * QD;
    } else if (key < fp.n_keys) {
      src = poolb + (static_cast<size_t>(fp.b) * a.N_cap + key - fp.n_win) * QD;
    } else {  // masked filler rows: the first row of the pair's own query (in bounds, finite)
      src = qbase + (static_cast<size_t>(fp.b) * a.T + fp.t0) * QH * QD;
    }
    dma_row(src, lds + (n_issued % NRING) * TILEB + r * ROWB, fvoff[i]);
  };
  auto advance_fill = [&]() {
    ++n_issued;
    if (++ft >= fp.n_tiles) {
      ft = 0;
      if (++fj >= n_mine) {
        fmore = false;
      } else {
        fp = pair_of(a, item_of(fj), per_seq);
      }
    }
  };
  auto issue_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_row(i);
    advance_fill();
  };

  // ---------------------------------------------------------------- compute state
  constexpr int NKS = QD / 16;  // 16-channel steps of QK^T
  dbf16x8_t qf[NKS];            // B operand: head `head`, channels 16 ks + 8 half .. + 7
  df32x16_t o[QD / 32];         // O^T blocks: channels 32 cb + 8 q + 4 half + 0..3, head `head`
  const float c2 = a.scale * kLog2e;
  const float sink2 = a.sink[head] * kLog2e;
  // Q loads are inline asm: the compiler's wait analysis does not track them, so it puts no
  // vector-memory waits among the QK^T instructions that read Q (tracked loads issued in a
  // pair's last step stayed pending at the loop head in its analysis, and its waits there
  // drained the tile loads in flight every step).  Every load is waited for explicitly
  // (vmcnt(0)) before Q is read; the registers stay live (Q is read every step), so nothing
  // else is allocated to them while the loads are in flight.
  dsu32x4_t q_rs;  // descriptor of the Q rows being loaded
  auto q_setup = [&](const Pair& d) {
    const Seen sq = seen_of(a, d, qsel);
    const unsigned long long base =
        reinterpret_cast<unsigned long long>(qbase + (static_cast<size_t>(d.b) * a.T + sq.t) * QH * QD);
    q_rs[0] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(base));
    q_rs[1] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(base >> 32)) & 0xFFFFu;
    q_rs[2] = QH * QD * 2;
    q_rs[3] = kWord3;
  };
  auto q_load = [&](int ks) {
    const unsigned off = static_cast<unsigned>(head * ROWB + half * 16);
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen offset:%3"
                 : "=v"(qf[ks])
                 : "v"(off), "s"(q_rs), "i"(ks * 32)
                 : "memory");
  };
  auto load_q = [&](const Pair& d) {
    q_setup(d);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) q_load(ks);
  };
  // lane i < R/2: frequency of rotary pair i, loaded once (a load inside the loop would be
  // waited for together with the tile loads in flight)
  const double fq = lane < R / 2 ? a.inv_freq[lane] : 0.0;
  auto rope_table = [&](long long p) {
    if (R == 0) return;
    if (lane < R / 2) {
      const double turns = static_cast<double>(p + a.pos_off) * fq * kTurn;
      const float fr = static_cast<float>(turns - rint(turns));
      rtab[lane] = make_float2(__builtin_amdgcn_cosf(fr), __builtin_amdgcn_sinf(fr));
    }
  };
  auto rotate_q = [&]() {
    if (R == 0) return;
#pragma unroll
    for (int ks = NKS - R / 16; ks < NKS; ++ks) {
      const int pr0 = (16 * ks + 8 * half - (QD - R)) >> 1;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float2 cs = rtab[pr0 + i / 2];
        const float xv = static_cast<float>(qf[ks][i]), yv = static_cast<float>(qf[ks][i + 1]);
        qf[ks][i] = static_cast<__bf16>(xv * cs.x - yv * cs.y);
        qf[ks][i + 1] = static_cast<__bf16>(xv * cs.y + yv * cs.x);
      }
    }
  };
  // A operand of QK^T (key rows of the tile, channel step ks): row l32, chunk 2 ks + half
  const int kaddr0 = l32 * ROWB + ((half ^ dswz(l32)) << 4);
  // V^T fragments (channel block cb, key half kh): transposing reads of rows
  // 16 kh + 4 half + i (lo) and + 8 (hi); see the score/value layout note above
  int tr_lo, tr_hi;
  {
    const int n16 = lane & 15, dh = (lane >> 4) & 1;
    const int i = n16 >> 2, j = 2 * dh + ((n16 & 3) >> 1);
    const int common = 64 * i + (n16 & 1) * 8;
    tr_lo = (4 * half + i) * ROWB + common + 16 * (j ^ half);
    tr_hi = (4 * half + i + 8) * ROWB + common + 16 * (j ^ (half | 2));
  }
  auto vfrag = [&](const unsigned char* tb, int cb, int kh) {
    const unsigned char* vb = tb + 16 * kh * ROWB + 256 * (cb >> 2);
    const int x = 64 * (cb & 3);
    int olo, ohi;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(olo) : "v"(tr_lo), "s"(x));
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(ohi) : "v"(tr_hi), "s"(x));
    const di16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dlds_i16x4*)(vb + olo));
    const di16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dlds_i16x4*)(vb + ohi));
    return __builtin_bit_cast(dbf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  if (n_mine <= 0) return;
  // prologue: three tiles in flight, then the first pair's Q
  issue_tile();
  if (fmore) issue_tile();
  if (fmore) issue_tile();
  int cj = 0, ct = 0;  // compute cursor: item rank, tile
  Pair cp = pair_of(a, item_of(0), per_seq);
  Seen cs = seen_of(a, cp, qsel);
  load_q(cp);
  rope_table(cs.p);
  // Q is complete before the loop (and again at the end of each pair's last step): the
  // compiler's wait analysis then sees no Q load pending at the loop head, and puts no
  // vector-memory waits among the QK^T instructions (which would drain the tile loads in
  // flight every step)
  wait_vm<0>();
  bool q_fresh = true;  // Q of the current pair still to be rotated
  float m_run = sink2, l_run = 1.f;
#pragma unroll
  for (int cb = 0; cb < QD / 32; ++cb) {
    zero_acc(o[cb]);
  }

  for (int s = 0;; ++s) {
    // tile s has landed once at most 8 * (tiles issued after it) tile loads remain; the Q
    // loads and output stores issued in between only make the wait longer
    const int after = n_issued - 1 - s;
    if (after >= 2) wait_vm<16>();
    else if (after == 1) wait_vm<8>();
    else wait_vm<0>();
    tile_barrier();  // every wave's rows of tile s are in LDS; tile s - 1's buffer is free
    // tile s + 3 goes into the buffer of tile s - 1, one row every fourth QK^T instruction: a
    // wave's vector-memory issue stalls for ~200 cycles per 1 KB row, which a burst of eight
    // would add to the step; between matrix instructions it overlaps them
    const bool fill = fmore;
    if (q_fresh) {
      rotate_q();
      q_fresh = false;
    }
    const unsigned char* tb = lds + (s % NRING) * TILEB;
    const bool last = ct + 1 == cp.n_tiles;

    // S^T = K . Q^T over the tile's 32 keys
    df32x16_t sacc;
    constexpr int PF = 4;
    dbf16x8_t kr[PF];
    auto kfrag = [&](int ks) {
      // the XOR is formed at each read (volatile asm is not hoisted): 32 pre-XOR-ed offsets
      // kept live would not fit beside Q and the accumulators
      int off;
      asm volatile("v_xor_b32 %0, %1, %2" : "=v"(off) : "v"(kaddr0), "s"(ks << 5));
      return *reinterpret_cast<const dbf16x8_t*>(tb + off);
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) kr[i] = kfrag(i);
    asm volatile("s_nop 4" ::: "memory");  // Q may have just been rotated by VALU
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const dbf16x8_t kf = kr[ks % PF];
      if (ks + PF < NKS) kr[ks % PF] = kfrag(ks + PF);
      if (ks == 0) qk_mfma_first(sacc, kf, qf[ks]);
      else qk_mfma(sacc, kf, qf[ks]);
      if ((ks & 3) == 1 && fill) issue_row(ks >> 2);
      __builtin_amdgcn_sched_barrier(0);  // keeps the fragment reads PF ahead, not all hoisted
    }
    if (fill) advance_fill();
    drain_mfma();  // the softmax reads S^T
    // online softmax: this lane holds keys 8 (e / 4) + 4 half + e % 4 of the tile, for `head`
    const int g0 = ct * TK;
    const bool full = (g0 >= cs.glo && g0 + TK <= cs.ghi) || (g0 >= cp.n_win && g0 + TK <= cs.pend);
    float sv[16];
    float tmax = -INFINITY;
    if (full) {  // uniform: most tiles
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        sv[e] = sacc[e] * c2;
        tmax = fmaxf(tmax, sv[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = g0 + 8 * (e >> 2) + 4 * half + (e & 3);
        // branch-free: unsigned range tests, bitwise or
        const bool vis = (static_cast<unsigned>(key - cs.glo) < static_cast<unsigned>(cs.ghi - cs.glo)) |
                         (static_cast<unsigned>(key - cp.n_win) < static_cast<unsigned>(cs.pend - cp.n_win));
        sv[e] = vis ? sacc[e] * c2 : -INFINITY;
        tmax = fmaxf(tmax, sv[e]);
      }
    }
    tmax = swap_max(tmax);
    const float m_new = tmax > m_run + kLazyMax ? tmax : m_run;
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < QD / 32; ++cb) scale_acc(o[cb], alpha);
      drain_mfma();
    }
    m_run = m_new;
    float pe[16], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pe[e] = __builtin_amdgcn_exp2f(sv[e] - m_new);
      psum += pe[e];
    }
    l_run += swap_sum(psum);
    dbf16x8_t pb[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[kh][i] = static_cast<__bf16>(pe[8 * kh + i]);
    // O^T += V^T . P^T, key half by key half (an accumulator block is used again 16
    // instructions later, never back to back)
    // O^T += V^T . P^T, key half by key half (an accumulator block is used again 16
    // instructions later, never back to back).  In a pair's last step the next pair's Q (this
    // pair's again after the last) streams in, one load per matrix instruction.  (One copy of
    // the loop with the loads under a uniform branch: two copies, with and without the loads,
    // made the register allocator move the accumulators between register files.)
    auto pv_tile = [&]() {
      constexpr int VPF = 2;
      dbf16x8_t vr[VPF];
#pragma unroll
      for (int i = 0; i < VPF; ++i) vr[i] = vfrag(tb, i & 15, i >> 4);
      asm volatile("s_nop 4" ::: "memory");  // P^T was just written by VALU
#pragma unroll
      for (int st = 0; st < QD / 16; ++st) {  // st = 16 kh + cb
        const dbf16x8_t vf = vr[st % VPF];
        if (st + VPF < QD / 16) vr[st % VPF] = vfrag(tb, (st + VPF) & 15, (st + VPF) >> 4);
        pv_mfma(o[st & 15], vf, pb[st >> 4]);
        if (last) q_load(st);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (last) q_setup(pair_of(a, item_of(min(cj + 1, n_mine - 1)), per_seq));
    pv_tile();
    if (last) wait_vm<0>();
    if (!last) {
      ++ct;
      continue;
    }
    drain_mfma();
    // epilogue: normalise, counter-rotate the rope slice (eq. 26), store bf16.  A 32-lane
    // swap gives each lane 8 consecutive channels (16-byte stores).
    if (cp.two || qsel == 0) {
      const float inv = 1.f / l_run;
      const drsrc_t ors = rs_of(static_cast<bf16_t*>(a.out) + (static_cast<size_t>(cp.b) * a.T + cs.t) * QH * QD,
                                QH * QD * 2);
      const unsigned ob = static_cast<unsigned>((head * QD + half * 8) * 2);
#pragma unroll
      for (int cb = 0; cb < QD / 32; ++cb) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          unsigned w[2][2];
#pragma unroll
          for (int g2 = 0; g2 < 2; ++g2) {
            const int gq = 2 * gp + g2;
            float v[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) v[jj] = acc_read(o[cb][gq * 4 + jj]) * inv;
            const int ch0 = 32 * cb + 8 * gq;  // + 4 half: this lane's 4 channels
            if (R > 0 && ch0 >= QD - R) {
#pragma unroll
              for (int i2 = 0; i2 < 2; ++i2) {
                const float2 t = rtab[((ch0 - (QD - R)) >> 1) + 2 * half + i2];
                const float c = t.x, sn = -t.y;
                const float xv = v[2 * i2], yv = v[2 * i2 + 1];
                v[2 * i2] = xv * c - yv * sn;
                v[2 * i2 + 1] = xv * sn + yv * c;
              }
            }
            w[g2][0] = pack_bf16x2(v[0], v[1]);
            w[g2][1] = pack_bf16x2(v[2], v[3]);
          }
          const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
          du32x4_t val;
          val[0] = s0[0];
          val[1] = s1[0];
          val[2] = s0[1];
          val[3] = s1[1];
          __builtin_amdgcn_raw_buffer_store_b128(val, ors, ob + static_cast<unsigned>((32 * cb + 16 * gp) * 2), 0, 0);
        }
      }
    }
    if (++cj >= n_mine) break;
    ct = 0;
    cp = pair_of(a, item_of(cj), per_seq);
    cs = seen_of(a, cp, qsel);
    rope_table(cs.p);
    q_fresh = true;
    m_run = sink2;
    l_run = 1.f;
#pragma unroll
    for (int cb = 0; cb < QD / 32; ++cb) {
      zero_acc(o[cb]);
    }
  }
  wait_vm<0>();
}

bool attend_dense_fits(const AttendArgs& a) {
  // 32-bit buffer offsets into one sequence's window and pool rows
  constexpr long long kMaxRows = (1LL << 22) - 8;
  return !a.csa && a.dtype == 1 && a.H == QH && a.D == QD && (a.r == 0 || a.r == 64) && a.S_kv <= kMaxRows &&
         a.N_cap <= kMaxRows;
}

template <int R>
static hipError_t launch_dense(const AttendArgs& a, hipStream_t st) {
  static bool attr_set = false;
  static int n_cu = 0;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_dense_kernel<R>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kDenseLds);
    if (e != hipSuccess) return e;
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n_cu < 1) n_cu = 1;
    attr_set = true;
  }
  const long long n_items = static_cast<long long>(a.B) * ((a.T + 1) / 2);
  const unsigned blocks = static_cast<unsigned>(n_items < n_cu ? n_items : n_cu);
  hipLaunchKernelGGL((attend_dense_kernel<R>), dim3(blocks), dim3(256), kDenseLds, st, a);
  return hipGetLastError();
}

hipError_t launch_attend_dense(const AttendArgs& a, hipStream_t st) {
  return a.r == 64 ? launch_dense<64>(a, st) : launch_dense<0>(a, st);
}

}  // namespace dsv4
