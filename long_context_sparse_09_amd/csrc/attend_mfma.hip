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
// One workgroup = one query (all 64 heads), 4 wavefronts.  Wave (hb, kh) owns heads
// [32hb, 32hb+32); it scores key half kh of every 64-key tile and accumulates output
// channels [256kh, 256kh+256):
//   * the tile's key rows are gathered (window rows, then selected / visible pool rows) into
//     LDS with direct global->LDS loads, double-buffered so the next gather overlaps compute;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (A = 32 key rows from LDS, B = the wave's
//     rotated Q held in registers for the whole kernel); each lane then holds 16 keys of ONE
//     head, so the online-softmax max / sum need one cross-half shuffle;
//   * the two waves of a head block swap their tile maxima and P fragments through LDS, so
//     both run the same online softmax over all 64 keys (state seeded by the sink: max = s_h,
//     sum = 1, value 0);
//   * the S^T accumulator layout is exactly the B operand of O^T = V^T . P^T, so P goes from
//     accumulator to operand without a shuffle; V^T (A operand) is read from the same
//     row-major tile with ds_read_tr16_b64 (4x16 transposing LDS reads): K = V is stored once;
//   * the epilogue divides by the softmax sum, applies the counter-rotation and stores bf16.
#include "common.h"
#include "launch.h"

namespace dsv4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

namespace {

constexpr int AH = 64;                       // query heads
constexpr int AD = 512;                      // head_dim
constexpr int ANK = 64;                      // keys per tile
constexpr int APITCH = AD * 2 + 16;          // LDS bytes per key row (16 B pad)
constexpr int ATILE = ANK * APITCH;          // bytes per tile buffer
constexpr int ATILES_BYTES = 2 * ATILE;      // double buffer
constexpr int AXCH_BYTES = 2 * 2 * 2 * 64 * 16 + 2 * 2 * 64 * 4 * 2;  // P fragments, max, sum
constexpr float kLazy = 8.f;  // log2-domain headroom before the running max moves

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

__device__ __forceinline__ bf16x8_t pack8(const float (&v)[8]) {
  bf16x8_t r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(v[i]);
  return r;
}

}  // namespace

template <bool CSA>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
attend_mfma_kernel(AttendArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* tiles = lds;
  bf16x8_t* xp = reinterpret_cast<bf16x8_t*>(lds + ATILES_BYTES);    // [hb][kh][ss][lane]
  float* xmax = reinterpret_cast<float*>(lds + ATILES_BYTES + 2 * 2 * 2 * 64 * 16);  // [hb][kh][lane]
  float* xsum = xmax + 2 * 2 * 64;                                    // [hb][kh][lane]
  int* klist = reinterpret_cast<int*>(lds + ATILES_BYTES + AXCH_BYTES);  // CSA: selected rows
  __shared__ float rope_c[kMaxRope / 2], rope_s[kMaxRope / 2];  // at the query's position
  __shared__ int wave_tot[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int hb = wave & 1, kh = wave >> 1;

  // later queries see more keys: schedule them first
  const int qid = gridDim.x - 1 - blockIdx.x;
  const int b = qid / a.T, t = qid % a.T;
  const long long p = static_cast<long long>(a.q_pos0[b]) + t;
  const double qpos = static_cast<double>(p + a.pos_off);
  if (tid < a.r / 2) {  // one (cos, sin) per rotary pair, formed in double precision
    const double inv_freq = pow(a.theta, -2.0 * tid / a.r);
    double sn, cs;
    sincos(qpos * inv_freq, &sn, &cs);
    rope_c[tid] = static_cast<float>(cs);
    rope_s[tid] = static_cast<float>(sn);
  }

  // ---- key set: window rows [r0, r1) of kv_win, then compressed entries ----
  const long long lo = max(0LL, p - a.window + 1);
  const int r0 = static_cast<int>(max(lo - a.kv_pos0[b], 0LL));
  const int r1 = static_cast<int>(min(p + 1 - a.kv_pos0[b], static_cast<long long>(a.S_kv)));
  const int n_win = max(0, r1 - r0);
  int n_cmp;
  if constexpr (CSA) {
    const int* idx = a.topk_idx + (static_cast<size_t>(b) * a.T + t) * a.k;
    int base = 0;
    for (int c0 = 0; c0 < a.k; c0 += 256) {
      const int i = c0 + tid;
      const int e = i < a.k ? idx[i] : -1;
      const bool v = e >= 0 && e < a.N_cap;
      int tot;
      const int pos = base + block_excl_count<256>(v, &tot, wave_tot);
      if (v) klist[pos] = e;
      base += tot;
    }
    n_cmp = base;
  } else {
    long long v = a.N_cap > 0 ? (p + 1) / a.m_hca : 0;
    v = min(v, static_cast<long long>(a.n_pool ? a.n_pool[b] : a.N_cap));
    v = min(v, static_cast<long long>(a.N_cap));
    n_cmp = static_cast<int>(max(v, 0LL));
  }
  __syncthreads();  // klist, rope table
  const int n_keys = n_win + n_cmp;
  const int n_tiles = (n_keys + ANK - 1) / ANK;

  const bf16_t* win = static_cast<const bf16_t*>(a.kv_win) + static_cast<size_t>(b) * a.S_kv * AD;
  const bf16_t* pool = static_cast<const bf16_t*>(a.pool) + static_cast<size_t>(b) * a.N_cap * AD;
  // Row of key x; keys past the end of a partial tile load key 0 (finite data, masked below).
  auto key_row = [&](int x) -> const bf16_t* {
    if (x >= n_keys) x = 0;
    if (x < n_win) return win + static_cast<size_t>(r0 + x) * AD;
    const int e = CSA ? klist[x - n_win] : x - n_win;
    return pool + static_cast<size_t>(e) * AD;
  };
  // Gather tile `it` into buffer `buf`: each wave instruction moves one 1 KB key row.
  auto issue_tile = [&](int it, int buf) {
    unsigned char* tb = tiles + buf * ATILE;
#pragma unroll
    for (int pass = 0; pass < ANK / 4; ++pass) {
      const int row = pass * 4 + wave;
      const bf16_t* src = key_row(it * ANK + row) + lane * 8;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                       (lds_void*)(tb + row * APITCH), 16, 0, 0);
    }
  };
  if (n_tiles > 0) issue_tile(0, 0);

  // ---- rotated Q^T fragments (B operand): head hb*32 + l32, dims ks*16 + half*8 .. +8 ----
  const int rope0 = AD - a.r;  // first rotary channel
  bf16x8_t qf[AD / 16];
  {
    const bf16_t* qrow = static_cast<const bf16_t*>(a.q) +
                         ((static_cast<size_t>(b) * a.T + t) * AH + hb * 32 + l32) * AD + half * 8;
#pragma unroll
    for (int ks = 0; ks < AD / 16; ++ks) {
      const int c0 = ks * 16 + half * 8;
      if (c0 + 8 > rope0) {
        float v[8];
        Chunk<bf16_t>::load<8>(qrow + ks * 16, v);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          if (c0 + i >= rope0) {
            const int pr = (c0 + i - rope0) >> 1;
            const float c = rope_c[pr], sn = rope_s[pr], x = v[i], y = v[i + 1];
            v[i] = x * c - y * sn;
            v[i + 1] = x * sn + y * c;
          }
        }
        qf[ks] = pack8(v);
      } else {
        qf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + ks * 16));
      }
    }
  }

  const float c2 = a.scale * kLog2e;  // logits in the log2 domain
  const int head = hb * 32 + l32;
  // running reference max and softmax sum of this wave; both waves of a head block form the
  // full denominator for their own output channels, so both start from the sink (logit s_h,
  // value 0): max = s_h, sum = 1
  float m_run = a.sink[head] * kLog2e;
  float l_run = 1.f;
  constexpr int NDT = AD / 2 / 32;  // output channel tiles owned by this wave
  f32x16_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;

  // transposing-read lane geometry: group of 16 lanes = (half, dim-half dh); lane n of the
  // group supplies row n/4 and column chunk n%4 of a 4 x 16 block
  const int n16 = lane & 15, dh = (lane >> 4) & 1;
  const int tr_off = (n16 >> 2) * APITCH + (kh * (AD / 2) + dh * 16 + 4 * (n16 & 3)) * 2;
  const int xme = (hb * 2 + kh) * 64 + lane, xpa = (hb * 2 + (kh ^ 1)) * 64 + lane;

  for (int it = 0; it < n_tiles; ++it) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's gather of tile `it` has landed
    __syncthreads();                // ... and every wave's; buffer (it+1)&1 and xp are free
    if (it + 1 < n_tiles) issue_tile(it + 1, (it + 1) & 1);
    const unsigned char* tb = tiles + (it & 1) * ATILE;

    // S^T (32 keys of half kh x 32 heads) over the 512 channels; K fragments run 4 ahead
    f32x16_t s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    const unsigned char* arow = tb + (kh * 32 + l32) * APITCH + half * 16;
    {
      constexpr int PF = 4;
      bf16x8_t kr[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) kr[i] = *reinterpret_cast<const bf16x8_t*>(arow + i * 32);
#pragma unroll
      for (int ks = 0; ks < AD / 16; ++ks) {
        const bf16x8_t kf = kr[ks % PF];
        if (ks + PF < AD / 16) kr[ks % PF] = *reinterpret_cast<const bf16x8_t*>(arow + (ks + PF) * 32);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
      }
    }

    // online softmax over this wave's 32 keys (lane: head l32, keys (e/4)*8 + half*4 + e%4).
    // Each wave keeps its own reference max m_run and moves it only when a logit exceeds it
    // by more than 2^kLazy, so most tiles need no rescale of the accumulators.
    const int kbase = it * ANK + kh * 32 + half * 4;
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kbase + (e >> 2) * 8 + (e & 3);
      const float v = key < n_keys ? s[e] * c2 : -INFINITY;
      s[e] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = (tmax > m_run + kLazy) ? tmax : m_run;
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8_t pb[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = exp2f(s[e] - m_new);
      psum += pv;
      pb[e >> 3][e & 7] = static_cast<__bf16>(pv);
    }
    psum += __shfl_xor(psum, 32);
    xsum[xme] = psum;
    xmax[xme] = m_new;
    xp[(hb * 2 + kh) * 128 + lane] = pb[0];
    xp[(hb * 2 + kh) * 128 + 64 + lane] = pb[1];
    if (__ballot(m_new != m_run)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
    }
    m_run = m_new;
    __syncthreads();  // partner's P fragments, sum and reference max are in LDS
    // partner's P was formed against its own reference max: bring it to this wave's
    const float f = exp2f(xmax[xpa] - m_run);
    l_run = l_run * alpha + psum + xsum[xpa] * f;
    bf16x8_t px0 = xp[(hb * 2 + (kh ^ 1)) * 128 + lane];
    bf16x8_t px1 = xp[(hb * 2 + (kh ^ 1)) * 128 + 64 + lane];
    if (__ballot(f != 1.f)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        px0[e] = static_cast<__bf16>(static_cast<float>(px0[e]) * f);
        px1[e] = static_cast<__bf16>(static_cast<float>(px1[e]) * f);
      }
    }
    // B operands for k-steps 0..3 = keys 0..63 of the tile (half kh is this wave's own)
    const bf16x8_t pk[4] = {kh == 0 ? pb[0] : px0, kh == 0 ? pb[1] : px1,
                            kh == 0 ? px0 : pb[0], kh == 0 ? px1 : pb[1]};

    // O^T (32 channels x 32 heads per tile dt) += V^T (32 channels x 16 key slots) . P^T
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      const unsigned char* vbase = tb + (16 * ss + 4 * half) * APITCH + tr_off;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const unsigned char* va = vbase + dt * 64;
        const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(va));
        const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(va + 8 * APITCH));
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk[ss], o[dt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: normalise, counter-rotate (eq. 26), store channels [256kh, 256kh+256) ----
  const float inv = 1.f / l_run;
  bf16_t* orow = static_cast<bf16_t*>(a.out) + ((static_cast<size_t>(b) * a.T + t) * AH + head) * AD;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = o[dt][g * 4 + j] * inv;
      const int c0 = kh * (AD / 2) + dt * 32 + g * 8 + half * 4;
      if (c0 + 4 > rope0) {  // counter-rotation: the same angle, negated (eq. 26)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          if (c0 + i >= rope0) {
            const int pr = (c0 + i - rope0) >> 1;
            const float c = rope_c[pr], sn = rope_s[pr], x = v[i], y = v[i + 1];
            v[i] = x * c + y * sn;
            v[i + 1] = -x * sn + y * c;
          }
        }
      }
      Chunk<bf16_t>::store<4>(orow + c0, v);
    }
  }
}

bool attend_fast(int H, int D, int r, int dtype) {
  return dtype == 1 && H == AH && D == AD && r % 2 == 0 && r <= AD;
}

hipError_t launch_attend_generic(const AttendArgs& a, hipStream_t st);

template <bool CSA>
static hipError_t launch_mfma(const AttendArgs& a, hipStream_t st) {
  const size_t shmem = ATILES_BYTES + AXCH_BYTES + (CSA ? static_cast<size_t>(a.k) * sizeof(int) : 0);
  static bool attr_set = false;  // per instantiation; setting it again is harmless
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_mfma_kernel<CSA>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 158 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned blocks = static_cast<unsigned>(a.B) * a.T;
  hipLaunchKernelGGL((attend_mfma_kernel<CSA>), dim3(blocks), dim3(256), shmem, st, a);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  if (a.B == 0 || a.T == 0) return hipSuccess;
  if (attend_fast(a.H, a.D, a.r, a.dtype)) return a.csa ? launch_mfma<true>(a, st) : launch_mfma<false>(a, st);
  return launch_attend_generic(a, st);
}

}  // namespace dsv4
