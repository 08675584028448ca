// Compressor pooling (CSA overlapping windows / HCA disjoint windows) and the sliding-window
// RoPE copy, for gfx950.
//
// Source: DeepSeek-V4 model page (Transformers docs), "Hybrid attention (§2.3)" (CSA / HCA
// pools, sliding-window K=V branch, partial RoPE) and "Attention mask layout" (an entry covers
// the positions of its window and closes at the window's last token).
//
// Both kernels are HBM-bound streaming kernels: every thread owns VEC consecutive channels
// (16-byte loads for bf16 with VEC = 8) so that a wavefront reads whole contiguous rows.
#include "common.h"
#include "launch.h"

namespace dsv4 {

// ---------------------------------------------------------------------------
// compress: entry w, channel c = softmax_j(gate[j,c] + bias[slot,c]) weighted sum of x[j,c]
// over the window of w (reading R1/R2), then RoPE at (w+1)m - 1 (R5).
//
// Block layout: threads = E entries x P slot-groups x G channel-groups (G = C / VEC).
// Each thread runs an online softmax over its slot range; the P partial states of one
// (entry, channel group) are merged through LDS.  The online update uses one exp2 per
// element: of the old maximum and the new logit, exactly one is the new maximum.
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__global__ void __launch_bounds__(256) compress_kernel(
    const T* __restrict__ x, const T* __restrict__ gate, const T* __restrict__ x_prev,
    const T* __restrict__ gate_prev, const float* __restrict__ bias, T* __restrict__ pool, int S,
    int C, int m, int overlap, int e0, int e1, int N_cap, int r, const RopeFreq rf, long long pos_off,
    int G, int P, int E) {
  extern __shared__ float red[];  // [E*P*G][3*VEC] partial states when P > 1
  __shared__ double inv_freq[kMaxRope / 2];
  for (int i = threadIdx.x; i < r / 2; i += blockDim.x) inv_freq[i] = rf.inv[i];
  const int tid = threadIdx.x;
  const int g = tid % G;
  const int p = (tid / G) % P;
  const int e = tid / (G * P);
  const int b = blockIdx.y;
  const int w = e0 + blockIdx.x * E + e;
  const bool active = (e < E) && (w < e1);
  const int span = overlap ? 2 * m : m;
  const int lo = overlap ? (w - 1) * m : w * m;
  const int chunk = (span + P - 1) / P;
  const int s0 = p * chunk;
  const int s1 = min(span, s0 + chunk);
  const int c0 = g * VEC;

  float mx[VEC], sm[VEC], acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) { mx[i] = -INFINITY; sm[i] = 0.f; acc[i] = 0.f; }

  if (active) {
    const size_t row0 = static_cast<size_t>(b) * S;
    // Slots in groups of U: the row loads of a group (values, gates and the slot biases) are
    // all issued before any is used, so a thread keeps them in flight together instead of
    // paying one slot's latency at a time (a bias load issued at its use would make the wait
    // for it cover every load issued before it).
    constexpr int U = 8;
    for (int sg = s0; sg < s1; sg += U) {
      float xv[U][VEC], gv[U][VEC], bv[U][VEC];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = sg + u;
        const int j = lo + s;
        ok[u] = s < s1 && j >= 0 && j < S;
        const size_t jr = row0 + (ok[u] ? j : 0);  // a valid row; unused when !ok
        // the earlier half of a window reads the second projection when one is given
        const bool early = x_prev != nullptr && s < m;
        Chunk<T>::template load<VEC>((early ? x_prev : x) + jr * C + c0, xv[u]);
        Chunk<T>::template load<VEC>((early ? gate_prev : gate) + jr * C + c0, gv[u]);
        if (bias != nullptr)
          Chunk<float>::template load<VEC>(bias + static_cast<size_t>(ok[u] ? s : 0) * C + c0, bv[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!ok[u]) continue;
        if (bias != nullptr) {
#pragma unroll
          for (int i = 0; i < VEC; ++i) gv[u][i] += bv[u][i];
        }
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float a = gv[u][i] * kLog2e;
          const float d = exp2f(-fabsf(a - mx[i]));  // 0 on the first slot (mx = -inf)
          if (a > mx[i]) {
            sm[i] = sm[i] * d + 1.f;
            acc[i] = acc[i] * d + xv[u][i];
            mx[i] = a;
          } else {
            sm[i] += d;
            acc[i] += d * xv[u][i];
          }
        }
      }
    }
  }

  __syncthreads();  // inv_freq staged
  if (P > 1) {
    float* mine = red + static_cast<size_t>(tid) * 3 * VEC;
#pragma unroll
    for (int i = 0; i < VEC; ++i) { mine[i] = mx[i]; mine[VEC + i] = sm[i]; mine[2 * VEC + i] = acc[i]; }
    __syncthreads();
    if (p == 0) {
      for (int q = 1; q < P; ++q) {
        const float* o = red + static_cast<size_t>(tid + q * G) * 3 * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float om = o[i];
          if (om == -INFINITY) continue;
          const float nm = fmaxf(mx[i], om);
          const float fa = exp2f(mx[i] - nm), fb = exp2f(om - nm);
          sm[i] = sm[i] * fa + o[VEC + i] * fb;
          acc[i] = acc[i] * fa + o[2 * VEC + i] * fb;
          mx[i] = nm;
        }
      }
    }
  }
  if (!active || p != 0) return;

  float out[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) out[i] = acc[i] / sm[i];
  const double pos = static_cast<double>((static_cast<long long>(w) + 1) * m - 1 + pos_off);
  rope_chunk<VEC, sizeof(T) == 2>(out, c0, C, r, pos, inv_freq);
  Chunk<T>::template store<VEC>(pool + (static_cast<size_t>(b) * N_cap + w) * C + c0, out);
}

template <typename T, int VEC>
static hipError_t compress_t(const void* x, const void* gate, const void* x_prev, const void* gate_prev,
                             const float* bias, void* pool, int B, int S, int C, int m, int overlap, int e0,
                             int e1, int N_cap, int r, double theta, long long off, hipStream_t st) {
  const int G = C / VEC;
  const int span = overlap ? 2 * m : m;
  // long windows: split the slots over P thread groups (16+ slots each)
  int P = 1;
  if (span >= 32) P = max(1, min(256 / G, span / 16));
  const int E = max(1, 256 / (G * P));
  const int threads = G * P * E;
  const int n = e1 - e0;
  if (n <= 0) return hipSuccess;
  dim3 grid(div_up(n, E), B);
  size_t shmem = P > 1 ? static_cast<size_t>(threads) * 3 * VEC * sizeof(float) : 0;
  hipLaunchKernelGGL((compress_kernel<T, VEC>), grid, dim3(threads), shmem, st,
                     static_cast<const T*>(x), static_cast<const T*>(gate), static_cast<const T*>(x_prev),
                     static_cast<const T*>(gate_prev), bias, static_cast<T*>(pool), S, C, m, overlap, e0, e1,
                     N_cap, r,
                     make_rope_freq(r, theta), off, G, P, E);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// compress, overlapping windows at a small rate (CSA, m = M, bf16, VEC = 8 channels a lane):
// register-resident windows.  The tokens of an entry's window form two blocks of M tokens,
// [(w-1)M, wM) (slots 0..M-1) and [wM, (w+1)M) (slots M..2M-1), and each block belongs to two
// consecutive entries.  A stream (the G = C/8 lanes of one row) pools E consecutive entries:
// it loads its E + 1 blocks once, all up front, so every token is read from memory once per
// stream (neighbouring streams share one block, fetched into the same XCD's L2: consecutive
// streams are dealt to one XCD), and keeps them in registers.  Per entry and channel the
// softmax is taken in two passes over the 2M slots (maximum, then exponentials), with the
// slot biases pre-scaled to the log2 domain once per stream.  One wavefront per block, no
// barriers besides the RoPE table's.
// ---------------------------------------------------------------------------
template <int M, int E>
__global__ void __launch_bounds__(64) compress_window_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ gate, const float* __restrict__ bias,
    bf16_t* __restrict__ pool, int S, int C, int e0, int e1, int N_cap, int r, const RopeFreq rf,
    long long pos_off, int G, int n_streams, int blocks_per_xcd) {
  constexpr int VEC = 8;
  constexpr int NB = E + 1;  // token blocks of a stream
  __shared__ double inv_freq[kMaxRope / 2];
  for (int i = threadIdx.x; i < r / 2; i += 64) inv_freq[i] = rf.inv[i];
  __syncthreads();
  // consecutive logical blocks on one XCD (the hardware deals workgroups to XCDs round-robin)
  const int lb = (blockIdx.x % 8) * blocks_per_xcd + blockIdx.x / 8;
  const int spb = 64 / G;  // streams per block
  const int stream = lb * spb + static_cast<int>(threadIdx.x) / G;
  if (stream >= n_streams || static_cast<int>(threadIdx.x) >= spb * G) return;
  const int g = static_cast<int>(threadIdx.x) % G;
  const int c0 = g * VEC;
  const int b = blockIdx.y;
  const int w0 = e0 + stream * E;
  const int n_e = min(E, e1 - w0);

  // all token rows of the stream's blocks: block k covers tokens (w0 - 1 + k) M .. + M - 1
  uint4 xr[NB][M], gr[NB][M];
  const bf16_t* xb = x + static_cast<size_t>(b) * S * C + c0;
  const bf16_t* gb = gate + static_cast<size_t>(b) * S * C + c0;
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int j = (w0 - 1 + k) * M + i;
      const bool ok = j >= 0 && k <= n_e;
      const size_t jr = static_cast<size_t>(ok ? j : 0) * C;
      xr[k][i] = *reinterpret_cast<const uint4*>(xb + jr);
      gr[k][i] = *reinterpret_cast<const uint4*>(gb + jr);
    }
  // slot biases, log2 domain: every slot's loads are issued before any is scaled (scaling each
  // slot as it arrives made every later slot's loads wait a memory round trip)
  float bz[2 * M][VEC];
  if (bias != nullptr) {
#pragma unroll
    for (int s2 = 0; s2 < 2 * M; ++s2)
      Chunk<float>::template load<VEC>(bias + static_cast<size_t>(s2) * C + c0, bz[s2]);
#pragma unroll
    for (int s2 = 0; s2 < 2 * M; ++s2)
#pragma unroll
      for (int i = 0; i < VEC; ++i) bz[s2][i] *= kLog2e;
  } else {
#pragma unroll
    for (int s2 = 0; s2 < 2 * M; ++s2)
#pragma unroll
      for (int i = 0; i < VEC; ++i) bz[s2][i] = 0.f;
  }
  auto unpack = [](const uint4& u, float (&v)[VEC]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  };
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e >= n_e) break;
    const int w = w0 + e;
    float out[VEC];
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch) out[ch] = 0.f;
    // logits of the 2M slots (block e: slots 0..M-1, absent before token 0; block e+1: M..2M-1)
    float a[2 * M][VEC];
    float mx[VEC];
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch) mx[ch] = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < 2 * M; ++s2) {
      float gv[VEC];
      unpack(gr[e + s2 / M][s2 % M], gv);
      const bool present = (w - 1) * M + s2 >= 0;
#pragma unroll
      for (int ch = 0; ch < VEC; ++ch) {
        a[s2][ch] = present ? fmaf(gv[ch], kLog2e, bz[s2][ch]) : -INFINITY;
        mx[ch] = fmaxf(mx[ch], a[s2][ch]);
      }
    }
    float sum[VEC], acc[VEC];
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch) { sum[ch] = 0.f; acc[ch] = 0.f; }
#pragma unroll
    for (int s2 = 0; s2 < 2 * M; ++s2) {
      float xv[VEC];
      unpack(xr[e + s2 / M][s2 % M], xv);
#pragma unroll
      for (int ch = 0; ch < VEC; ++ch) {
        const float p = __builtin_amdgcn_exp2f(a[s2][ch] - mx[ch]);  // 0 for absent slots
        sum[ch] += p;
        acc[ch] = fmaf(p, xv[ch], acc[ch]);
      }
    }
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch) out[ch] = acc[ch] * __builtin_amdgcn_rcpf(sum[ch]);
    const double pos = static_cast<double>((static_cast<long long>(w) + 1) * M - 1 + pos_off);
    rope_chunk<VEC, true>(out, c0, C, r, pos, inv_freq);
    Chunk<bf16_t>::template store<VEC>(pool + (static_cast<size_t>(b) * N_cap + w) * C + c0, out);
  }
}

// ---------------------------------------------------------------------------
// compress, overlapping windows (CSA, m = M, bf16, C a multiple of 128): LDS-staged.  A
// workgroup of WPB wavefronts pools NE = WPB * (64 / G) consecutive entries w0 .. w0 + NE - 1
// (G = C/8 lanes per entry, 8 channels a lane).  Their windows cover the contiguous token rows
// [(w0 - 1) M, (w0 + NE) M), one contiguous span of each input, which the workgroup first
// copies into LDS with straight 1 KB buffer loads (buffer_load ... lds): every token is read
// from memory once per workgroup (plus an M-row halo) instead of once per window that holds
// it, in fully coalesced 1 KB pieces.  Rows outside the sequence read as zeros; only absent
// slots (before token 0) or entries past e1 (not stored) touch them.  Each entry is then
// pooled from LDS as the register-window kernel pools it: two-pass softmax over the 2M slots
// with the slot biases in the log2 domain, RoPE epilogue.
// ---------------------------------------------------------------------------
template <int M, int WPB>
__global__ void __launch_bounds__(64 * WPB) compress_staged_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ gate, const float* __restrict__ bias,
    bf16_t* __restrict__ pool, int S, int C, int e0, int e1, int N_cap, int r, const RopeFreq rf,
    long long pos_off, int G, int n_blocks, int blocks_per_xcd) {
  constexpr int VEC = 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char stg[];  // [x | gate][rows][C] bf16
  __shared__ double inv_freq[kMaxRope / 2];
  for (int i = threadIdx.x; i < r / 2; i += 64 * WPB) inv_freq[i] = rf.inv[i];
  const int lb = (blockIdx.x % 8) * blocks_per_xcd + blockIdx.x / 8;  // consecutive blocks on one XCD
  if (lb >= n_blocks) return;  // block-uniform, before any barrier
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int NE = WPB * (64 / G);
  const int w0 = e0 + lb * NE;
  const int row_bytes = C * 2;
  const int span = (NE + 1) * M * row_bytes;  // bytes of one input's token span (a multiple of 1 KB)
  // the span starts at token (w0 - 1) M; offsets are taken from the sequence's first row, so
  // the rows before it (w0 = 0) have negative offsets, which wrap past the descriptor's end
  const int start = (w0 - 1) * M * row_bytes;
  const unsigned seq_bytes = static_cast<unsigned>(S) * static_cast<unsigned>(row_bytes);
  typedef __attribute__((address_space(3))) void lds_void_t;
  const __amdgpu_buffer_rsrc_t x_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(x + static_cast<size_t>(b) * S * C), static_cast<short>(0), static_cast<int>(seq_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t g_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(gate + static_cast<size_t>(b) * S * C), static_cast<short>(0), static_cast<int>(seq_bytes), 0x00020000);
  const int n_kb = span / 1024;
  for (int k = wave; k < n_kb; k += WPB) {
    const unsigned off = static_cast<unsigned>(start + k * 1024 + lane * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rs, (lds_void_t*)(stg + k * 1024), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(g_rs, (lds_void_t*)(stg + span + k * 1024), 16, off, 0, 0, 0);
  }
  // slot biases (log2 domain) while the span lands
  const int g = lane % G;
  const int c0 = g * VEC;
  float bz[2 * M][VEC];
  if (bias != nullptr) {
#pragma unroll
    for (int s2 = 0; s2 < 2 * M; ++s2)
      Chunk<float>::template load<VEC>(bias + static_cast<size_t>(s2) * C + c0, bz[s2]);
#pragma unroll
    for (int s2 = 0; s2 < 2 * M; ++s2)
#pragma unroll
      for (int i = 0; i < VEC; ++i) bz[s2][i] *= kLog2e;
  } else {
#pragma unroll
    for (int s2 = 0; s2 < 2 * M; ++s2)
#pragma unroll
      for (int i = 0; i < VEC; ++i) bz[s2][i] = 0.f;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
  __syncthreads();                     // and every wave's
  const int e = wave * (64 / G) + lane / G;  // this stream's entry within the block
  const int w = w0 + e;
  if (w >= e1 || lane >= (64 / G) * G) return;  // no barrier follows
  auto unpack = [](const uint4& u, float (&v)[VEC]) {
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(wd[i] << 16);
      v[2 * i + 1] = __uint_as_float(wd[i] & 0xffff0000u);
    }
  };
  // slot s2 of entry e is span row e M + s2
  const unsigned char* xs = stg + (e * M) * row_bytes + c0 * 2;
  const unsigned char* gs = xs + span;
  float a[2 * M][VEC];
  float mx[VEC];
#pragma unroll
  for (int ch = 0; ch < VEC; ++ch) mx[ch] = -INFINITY;
#pragma unroll
  for (int s2 = 0; s2 < 2 * M; ++s2) {
    float gv[VEC];
    unpack(*reinterpret_cast<const uint4*>(gs + s2 * row_bytes), gv);
    const bool present = (w - 1) * M + s2 >= 0;
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch) {
      a[s2][ch] = present ? fmaf(gv[ch], kLog2e, bz[s2][ch]) : -INFINITY;
      mx[ch] = fmaxf(mx[ch], a[s2][ch]);
    }
  }
  float sum[VEC], acc[VEC];
#pragma unroll
  for (int ch = 0; ch < VEC; ++ch) {
    sum[ch] = 0.f;
    acc[ch] = 0.f;
  }
#pragma unroll
  for (int s2 = 0; s2 < 2 * M; ++s2) {
    float xv[VEC];
    unpack(*reinterpret_cast<const uint4*>(xs + s2 * row_bytes), xv);
#pragma unroll
    for (int ch = 0; ch < VEC; ++ch) {
      const float p = __builtin_amdgcn_exp2f(a[s2][ch] - mx[ch]);  // 0 for absent slots
      sum[ch] += p;
      acc[ch] = fmaf(p, xv[ch], acc[ch]);
    }
  }
  float out[VEC];
#pragma unroll
  for (int ch = 0; ch < VEC; ++ch) out[ch] = acc[ch] * __builtin_amdgcn_rcpf(sum[ch]);
  const double pos = static_cast<double>((static_cast<long long>(w) + 1) * M - 1 + pos_off);
  rope_chunk<VEC, true>(out, c0, C, r, pos, inv_freq);
  Chunk<bf16_t>::template store<VEC>(pool + (static_cast<size_t>(b) * N_cap + w) * C + c0, out);
}

// ---------------------------------------------------------------------------
// compress, disjoint windows at a large rate (HCA, m = NG * GS slots, bf16, C = 512): one
// workgroup per entry, NG wavefronts; wavefront p pools slots [p GS, (p + 1) GS) for all 512
// channels (lane l owns channels 8l .. 8l + 7), in groups of 4 tokens.  The loads of group
// g + 1 (values, gates, slot biases) are issued before group g's arithmetic, so a wavefront
// always has a group in flight; HB (slot biases given) is a template parameter, so no load is
// conditional and the waits cover exactly the group about to be pooled.  A group is pooled in
// two passes (maximum, then exponentials) and merged into the wavefront's running state; the
// NG states of a channel are merged through LDS by wavefront 0, which also applies RoPE.
// ---------------------------------------------------------------------------
template <int NG, int GS, bool HB>
__global__ void __launch_bounds__(NG * 64) compress_disjoint_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ gate, const float* __restrict__ bias,
    bf16_t* __restrict__ pool, int S, int e0, int N_cap, int r, const RopeFreq rf, long long pos_off) {
  constexpr int C = 512, VEC = 8, M = NG * GS, U = 4;
  static_assert(GS % U == 0, "slot groups of 4");
  __shared__ float red[NG][3][VEC][64];  // per wavefront: max, sum, acc of each lane's channels
  __shared__ double inv_freq[kMaxRope / 2];
  for (int i = threadIdx.x; i < r / 2; i += NG * 64) inv_freq[i] = rf.inv[i];
  const int lane = threadIdx.x & 63, p = threadIdx.x >> 6;
  const int b = blockIdx.y, w = e0 + blockIdx.x;
  const int c0 = lane * VEC;
  const bf16_t* xb = x + (static_cast<size_t>(b) * S + static_cast<size_t>(w) * M) * C + c0;
  const bf16_t* gb = gate + (static_cast<size_t>(b) * S + static_cast<size_t>(w) * M) * C + c0;
  float mx[VEC], sm[VEC], acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) { mx[i] = -INFINITY; sm[i] = 0.f; acc[i] = 0.f; }
  auto unpack = [](const uint4& u, float (&v)[VEC]) {
    const uint32_t q[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  };
  uint4 xq[2][U], gq[2][U];
  float bq[2][U][VEC];
  auto load_group = [&](int s0, int k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xq[k][u] = *reinterpret_cast<const uint4*>(xb + static_cast<size_t>(s0 + u) * C);
      gq[k][u] = *reinterpret_cast<const uint4*>(gb + static_cast<size_t>(s0 + u) * C);
      if constexpr (HB) Chunk<float>::template load<VEC>(bias + static_cast<size_t>(s0 + u) * C + c0, bq[k][u]);
    }
  };
  load_group(p * GS, 0);
#pragma unroll
  for (int kg = 0; kg < GS / U; ++kg) {
    const int s0 = p * GS + kg * U;
    if (kg + 1 < GS / U) load_group(s0 + U, (kg + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);  // the next group's loads stay ahead of this fold
    const uint4 (&xr)[U] = xq[kg & 1];
    const uint4 (&gr)[U] = gq[kg & 1];
    const float (&bv)[U][VEC] = bq[kg & 1];
    float a[U][VEC], gm[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) gm[i] = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float gv[VEC];
      unpack(gr[u], gv);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        a[u][i] = (HB ? gv[i] + bv[u][i] : gv[i]) * kLog2e;
        gm[i] = fmaxf(gm[i], a[u][i]);
      }
    }
    // fold the group into the running state at the new maximum
    float nm[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      nm[i] = fmaxf(mx[i], gm[i]);
      const float f = __builtin_amdgcn_exp2f(mx[i] - nm[i]);  // 0 while the state is empty
      sm[i] *= f;
      acc[i] *= f;
      mx[i] = nm[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xv[VEC];
      unpack(xr[u], xv);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float e = __builtin_amdgcn_exp2f(a[u][i] - nm[i]);
        sm[i] += e;
        acc[i] = fmaf(e, xv[i], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    red[p][0][i][lane] = mx[i];
    red[p][1][i][lane] = sm[i];
    red[p][2][i][lane] = acc[i];
  }
  __syncthreads();
  if (p != 0) return;
  float out[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    float m_all = red[0][0][i][lane];
#pragma unroll
    for (int q = 1; q < NG; ++q) m_all = fmaxf(m_all, red[q][0][i][lane]);
    float s_all = 0.f, a_all = 0.f;
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const float f = __builtin_amdgcn_exp2f(red[q][0][i][lane] - m_all);
      s_all = fmaf(red[q][1][i][lane], f, s_all);
      a_all = fmaf(red[q][2][i][lane], f, a_all);
    }
    out[i] = a_all * __builtin_amdgcn_rcpf(s_all);
  }
  const double pos = static_cast<double>((static_cast<long long>(w) + 1) * M - 1 + pos_off);
  rope_chunk<VEC, true>(out, c0, C, r, pos, inv_freq);
  Chunk<bf16_t>::template store<VEC>(pool + (static_cast<size_t>(b) * N_cap + w) * C + c0, out);
}

hipError_t launch_compress(const void* x, const void* gate, const void* x_prev, const void* gate_prev,
                           const float* bias, void* pool, int B, int S, int C, int m, int overlap, int e0,
                           int e1, int N_cap, int r, double theta, long long off, int dtype, hipStream_t st) {
  const bool v8 = (C % 8 == 0) && (C / 8 <= 256);
  if (!overlap) x_prev = gate_prev = nullptr;  // no earlier half
  if (dtype == 1 && overlap && m == 4 && x_prev == nullptr && C % 128 == 0 && C <= 512 && 64 % (C / 8) == 0 &&
      e1 > e0 && static_cast<long long>(S) * C * 2 < (1LL << 31)) {
    // four entries per workgroup: one wavefront at C = 128 (four entries a wavefront), four
    // at C = 512, so that 2048 entries make 512 workgroups either way
    const int G = C / 8;
    const int wpb = C >= 512 ? 4 : (C >= 256 ? 2 : 1);
    const int NE = wpb * (64 / G);
    const int nb = static_cast<int>(div_up(static_cast<uint32_t>(e1 - e0), NE));
    const int per = static_cast<int>(div_up(static_cast<uint32_t>(nb), 8));
    const size_t lds = 2 * static_cast<size_t>(NE + 1) * 4 * C * 2;
    const RopeFreq rfq = make_rope_freq(r, theta);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* gb = static_cast<const bf16_t*>(gate);
    bf16_t* pb = static_cast<bf16_t*>(pool);
    if (wpb == 4)
      hipLaunchKernelGGL((compress_staged_kernel<4, 4>), dim3(8 * per, B), dim3(256), lds, st, xb, gb, bias, pb, S,
                         C, e0, e1, N_cap, r, rfq, off, G, nb, per);
    else if (wpb == 2)
      hipLaunchKernelGGL((compress_staged_kernel<4, 2>), dim3(8 * per, B), dim3(128), lds, st, xb, gb, bias, pb, S,
                         C, e0, e1, N_cap, r, rfq, off, G, nb, per);
    else
      hipLaunchKernelGGL((compress_staged_kernel<4, 1>), dim3(8 * per, B), dim3(64), lds, st, xb, gb, bias, pb, S,
                         C, e0, e1, N_cap, r, rfq, off, G, nb, per);
    return hipGetLastError();
  }
  if (dtype == 1 && overlap && m == 4 && x_prev == nullptr && C % 8 == 0 && C / 8 <= 64 &&
      64 % (C / 8) == 0 && e1 > e0) {
    constexpr int E = 1;  // entries per stream (1: twice the wavefronts of 2, measured faster)
    const int G = C / 8;
    const int n_streams = static_cast<int>(div_up(static_cast<uint32_t>(e1 - e0), E));
    const int nb = static_cast<int>(div_up(static_cast<uint32_t>(n_streams), 64 / G));
    const int per = static_cast<int>(div_up(static_cast<uint32_t>(nb), 8));
    hipLaunchKernelGGL((compress_window_kernel<4, E>), dim3(8 * per, B), dim3(64), 0, st,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(gate), bias,
                       static_cast<bf16_t*>(pool), S, C, e0, e1, N_cap, r, make_rope_freq(r, theta), off, G,
                       n_streams, per);
    return hipGetLastError();
  }
  if (dtype == 1 && !overlap && m == 128 && C == 512 && e1 > e0) {
    if (bias != nullptr)
      hipLaunchKernelGGL((compress_disjoint_kernel<8, 16, true>), dim3(e1 - e0, B), dim3(512), 0, st,
                         static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(gate), bias,
                         static_cast<bf16_t*>(pool), S, e0, N_cap, r, make_rope_freq(r, theta), off);
    else
      hipLaunchKernelGGL((compress_disjoint_kernel<8, 16, false>), dim3(e1 - e0, B), dim3(512), 0, st,
                         static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(gate), bias,
                         static_cast<bf16_t*>(pool), S, e0, N_cap, r, make_rope_freq(r, theta), off);
    return hipGetLastError();
  }
  if (dtype == 1) {
    return v8 ? compress_t<bf16_t, 8>(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r,
                                      theta, off, st)
              : compress_t<bf16_t, 2>(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r,
                                      theta, off, st);
  }
  return v8 ? compress_t<float, 8>(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r,
                                   theta, off, st)
            : compress_t<float, 2>(x, gate, x_prev, gate_prev, bias, pool, B, S, C, m, overlap, e0, e1, N_cap, r,
                                   theta, off, st);
}

// ---------------------------------------------------------------------------
// Compressor cache update (decode): one workgroup per sequence.  lengths[b] = L counts the
// sequence's tokens including the new one.  The new raw token (x_new[b], gate_new[b]) goes
// into ring slot (L-1) mod span of the sequence's token ring (span = 2m with overlap, m
// without); when it closes an entry (L mod m == 0, emit != 0), entry w = L/m - 1 is pooled
// from the ring exactly as compress_kernel pools it with P = 1 (same slot order, same
// online softmax) and rotated at (w+1)m - 1.  Each thread owns one channel chunk of both the
// store and the pooling, so it reads back its own write.
// ---------------------------------------------------------------------------
template <typename T, int VEC>
__device__ __forceinline__ void cache_update_body(
    const T* __restrict__ x_new, const T* __restrict__ g_new, T* x_ring, T* g_ring,
    const T* __restrict__ xp_new, const T* __restrict__ gp_new, T* xp_ring, T* gp_ring,
    const float* __restrict__ bias, T* __restrict__ pool, const int* __restrict__ lengths, int C,
    int m, int overlap, int N_cap, int r, const RopeFreq& rf, long long pos_off, int emit) {
  __shared__ double inv_freq[kMaxRope / 2];
  for (int i = threadIdx.x; i < r / 2; i += blockDim.x) inv_freq[i] = rf.inv[i];
  __syncthreads();
  const int b = blockIdx.x;
  const int L = lengths[b];
  if (L < 1) return;  // block-uniform; no barrier follows
  const int span = overlap ? 2 * m : m;
  const int G = C / VEC;
  const size_t ring0 = static_cast<size_t>(b) * span;
  const int slot = (L - 1) % span;
  const bool closes = emit && (L % m) == 0 && (L / m - 1) < N_cap;
  const int w = L / m - 1;
  const int lo = overlap ? (w - 1) * m : w * m;
  for (int g = threadIdx.x; g < G; g += blockDim.x) {
    const int c0 = g * VEC;
    // the new token's rows: every load before any store (each load waited for in turn cost a
    // memory round trip per row)
    const bool two = xp_ring != nullptr;  // the second projection, for the windows this token starts
    float v0[VEC], v1[VEC], v2[VEC], v3[VEC];
    Chunk<T>::template load<VEC>(x_new + static_cast<size_t>(b) * C + c0, v0);
    Chunk<T>::template load<VEC>(g_new + static_cast<size_t>(b) * C + c0, v1);
    Chunk<T>::template load<VEC>((two ? xp_new : x_new) + static_cast<size_t>(b) * C + c0, v2);
    Chunk<T>::template load<VEC>((two ? gp_new : g_new) + static_cast<size_t>(b) * C + c0, v3);
    Chunk<T>::template store<VEC>(x_ring + (ring0 + slot) * C + c0, v0);
    Chunk<T>::template store<VEC>(g_ring + (ring0 + slot) * C + c0, v1);
    if (two) {
      Chunk<T>::template store<VEC>(xp_ring + (ring0 + slot) * C + c0, v2);
      Chunk<T>::template store<VEC>(gp_ring + (ring0 + slot) * C + c0, v3);
    }
    if (!closes) continue;
    float mx[VEC], sm[VEC], acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) { mx[i] = -INFINITY; sm[i] = 0.f; acc[i] = 0.f; }
    // slots in batches of SB: a batch's loads are all issued, then its slots are folded into
    // the online softmax in slot order (the order compress_kernel uses)
    constexpr int SB = 4;
    for (int s0 = 0; s0 < span; s0 += SB) {
      float xv[SB][VEC], gv[SB][VEC], bv[SB][VEC];
      // loads are unconditional (slots past the span or before position 0 read a clamped,
      // valid row and are skipped below): a load under a branch is waited for inside it
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int s = min(s0 + j, span - 1);
        const int p = max(lo + s, 0);  // token position; absent before 0
        const size_t row = ring0 + p % span;
        const bool early = two && s < m;  // the earlier half's second projection
        Chunk<T>::template load<VEC>((early ? xp_ring : x_ring) + row * C + c0, xv[j]);
        Chunk<T>::template load<VEC>((early ? gp_ring : g_ring) + row * C + c0, gv[j]);
      }
      if (bias != nullptr) {
#pragma unroll
        for (int j = 0; j < SB; ++j)
          Chunk<float>::template load<VEC>(bias + static_cast<size_t>(min(s0 + j, span - 1)) * C + c0, bv[j]);
      }
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int s = s0 + j;
        if (s >= span || lo + s < 0) continue;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float a = (bias != nullptr ? gv[j][i] + bv[j][i] : gv[j][i]) * kLog2e;
          const float d = exp2f(-fabsf(a - mx[i]));
          if (a > mx[i]) {
            sm[i] = sm[i] * d + 1.f;
            acc[i] = acc[i] * d + xv[j][i];
            mx[i] = a;
          } else {
            sm[i] += d;
            acc[i] += d * xv[j][i];
          }
        }
      }
    }
    float out[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) out[i] = acc[i] / sm[i];
    const double pos = static_cast<double>((static_cast<long long>(w) + 1) * m - 1 + pos_off);
    rope_chunk<VEC, sizeof(T) == 2>(out, c0, C, r, pos, inv_freq);
    Chunk<T>::template store<VEC>(pool + (static_cast<size_t>(b) * N_cap + w) * C + c0, out);
  }
}

// One launch updates the compressors given (one, or two of one layer that share lengths, m,
// overlap and N_cap: the CSA K=V compressor and the indexer's); blockIdx.y picks the compressor,
// blockIdx.x the sequence.
template <typename T>
struct CacheLaunch {
  CacheUpdate u;
  int C, r;
  RopeFreq rf;
};

template <typename T, int VEC>
__global__ void __launch_bounds__(256) cache_update_kernel(const CacheLaunch<T> p0, const CacheLaunch<T> p1, int m,
                                                           int overlap, int N_cap, long long pos_off, int emit) {
  // one call per compressor on the kernel arguments themselves (selecting a reference to
  // either copied the argument block, rotary table included, into scratch memory)
  auto run = [&](const CacheLaunch<T>& p) {
    const CacheUpdate& u = p.u;
    cache_update_body<T, VEC>(static_cast<const T*>(u.x_new), static_cast<const T*>(u.g_new),
                              static_cast<T*>(u.x_ring), static_cast<T*>(u.g_ring), static_cast<const T*>(u.xp_new),
                              static_cast<const T*>(u.gp_new), static_cast<T*>(u.xp_ring),
                              static_cast<T*>(u.gp_ring), u.bias, static_cast<T*>(u.pool), u.lengths, p.C, m,
                              overlap, N_cap, p.r, p.rf, pos_off, emit);
  };
  if (blockIdx.y == 0) run(p0);
  else run(p1);
}

template <typename T, int VEC>
static hipError_t cache_update_t(const CacheUpdate* u, const int* C, const int* r, int n, int B, int m, int overlap,
                                 int N_cap, double theta, long long off, int emit, hipStream_t st) {
  CacheLaunch<T> p[2];
  int G = 1;
  for (int i = 0; i < n; ++i) {
    p[i] = CacheLaunch<T>{u[i], C[i], r[i], make_rope_freq(r[i], theta)};
    G = C[i] / VEC > G ? C[i] / VEC : G;
  }
  if (n == 1) p[1] = p[0];
  const int threads = G >= 256 ? 256 : ((G + 63) / 64) * 64;
  hipLaunchKernelGGL((cache_update_kernel<T, VEC>), dim3(B, n), dim3(threads), 0, st, p[0], p[1], m, overlap, N_cap,
                     off, emit);
  return hipGetLastError();
}

hipError_t launch_cache_update(const CacheUpdate* us, const int* Cs, const int* rs, int n, int B, int m, int overlap,
                               int N_cap, double theta, long long off, int emit, int dtype, hipStream_t st) {
  if (B == 0) return hipSuccess;
  CacheUpdate v[2];
  bool v8 = true;
  for (int i = 0; i < n; ++i) {
    v[i] = us[i];
    if (!overlap || v[i].xp_ring == nullptr) v[i].xp_new = v[i].gp_new = v[i].xp_ring = v[i].gp_ring = nullptr;
    v8 = v8 && (Cs[i] % 8 == 0) && (Cs[i] / 8 <= 256);
  }
  if (dtype == 1)
    return v8 ? cache_update_t<bf16_t, 8>(v, Cs, rs, n, B, m, overlap, N_cap, theta, off, emit, st)
              : cache_update_t<bf16_t, 2>(v, Cs, rs, n, B, m, overlap, N_cap, theta, off, emit, st);
  return v8 ? cache_update_t<float, 8>(v, Cs, rs, n, B, m, overlap, N_cap, theta, off, emit, st)
            : cache_update_t<float, 2>(v, Cs, rs, n, B, m, overlap, N_cap, theta, off, emit, st);
}

hipError_t launch_cache_update(const CacheUpdate& u, int B, int C, int m, int overlap, int N_cap, int r,
                               double theta, long long off, int emit, int dtype, hipStream_t st) {
  return launch_cache_update(&u, &C, &r, 1, B, m, overlap, N_cap, theta, off, emit, dtype, st);
}

// ---------------------------------------------------------------------------
// swa_concat: rotate raw K=V rows at their positions into the window buffer.
//
// The chunks of a row that hold no rotary channel (the first Gn of its G VEC-channel chunks)
// are a plain copy; the Gr = G - Gn trailing ones are rotated.  The grid is split in two
// regions so that no wavefront mixes the two kinds: blocks below nb_copy copy, the rest
// rotate (inv_freq staged in LDS).  Each thread handles SWA_U chunks a block-stride apart and
// issues all their loads before any store.  Index arithmetic is 32-bit (the host checks the
// chunk counts): 64-bit division is a long software sequence on this target.
// ---------------------------------------------------------------------------
constexpr int SWA_U = 4;

template <typename T, int VEC>
__global__ void __launch_bounds__(256) swa_kernel(const T* __restrict__ kv_raw, T* kv_win,
                                                  const int* __restrict__ kv_pos0,
                                                  const int* __restrict__ new_pos0, int S_new,
                                                  int S_cap, int D, int r, const RopeFreq rf,
                                                  long long pos_off, int Gn, unsigned n_copy,
                                                  unsigned n_rot, unsigned nb_copy) {
  __shared__ double inv_freq[kMaxRope / 2];
  const unsigned G = static_cast<unsigned>(D / VEC);
  const bool rot = blockIdx.x >= nb_copy;  // block-uniform
  const unsigned Gk = rot ? G - Gn : Gn;   // chunks of this kind per row
  const unsigned total = rot ? n_rot : n_copy;
  const unsigned blk = rot ? blockIdx.x - nb_copy : blockIdx.x;
  if (rot) {
    for (int i = threadIdx.x; i < r / 2; i += blockDim.x) inv_freq[i] = rf.inv[i];
    __syncthreads();
  }
  const unsigned base = blk * blockDim.x * SWA_U + threadIdx.x;
  // the chunks' rows, their sequences' start positions and their data are all requested
  // before any store, so the stores wait for one round trip, not one per chunk
  float v[SWA_U][VEC];
  unsigned rows[SWA_U];
  int np0[SWA_U], kp0[SWA_U];
#pragma unroll
  for (int u = 0; u < SWA_U; ++u) {
    const unsigned gid = base + u * blockDim.x;
    const unsigned ld = gid < total ? gid : total - 1;  // a valid chunk; unused past the end
    const unsigned row = ld / Gk;
    rows[u] = row;
    const unsigned g = (rot ? Gn : 0) + (ld - row * Gk);
    Chunk<T>::template load<VEC>(kv_raw + (static_cast<size_t>(row) * G + g) * VEC, v[u]);
    const unsigned b = row / static_cast<unsigned>(S_new);
    np0[u] = new_pos0[b];
    kp0[u] = kv_pos0[b];
  }
#pragma unroll
  for (int u = 0; u < SWA_U; ++u) {
    const unsigned gid = base + u * blockDim.x;
    if (gid >= total) break;
    const unsigned row = rows[u];  // b * S_new + i
    const int g = static_cast<int>((rot ? Gn : 0) + (gid - row * Gk));
    const int b = static_cast<int>(row / static_cast<unsigned>(S_new));
    const int i = static_cast<int>(row - static_cast<unsigned>(b) * S_new);
    const long long seq = static_cast<long long>(np0[u]) + i;
    const long long dst = seq - kp0[u];
    if (dst < 0 || dst >= S_cap) continue;
    if (rot)
      rope_chunk<VEC, sizeof(T) == 2>(v[u], g * VEC, D, r, static_cast<double>(seq + pos_off),
                                      inv_freq);
    Chunk<T>::template store<VEC>(kv_win + (static_cast<long long>(b) * S_cap + dst) * D + g * VEC,
                                  v[u]);
  }
}

template <typename T, int VEC>
static hipError_t swa_t(const void* kv_raw, void* kv_win, const int* kv_pos0, const int* new_pos0,
                        int B, int S_new, int S_cap, int D, int r, double theta, long long off,
                        hipStream_t st) {
  const long long rows = static_cast<long long>(B) * S_new;
  const int G = D / VEC;
  const int Gn = (D - r) / VEC;  // chunks with no rotary channel
  const long long n_copy = rows * Gn, n_rot = rows * (G - Gn);
  if (rows == 0) return hipSuccess;
  if (rows * G >= (1LL << 31)) return hipErrorInvalidValue;  // 32-bit chunk indices
  const int threads = 256;
  const long long per_block = static_cast<long long>(threads) * SWA_U;
  const long long nb_copy = (n_copy + per_block - 1) / per_block;
  const long long nb_rot = (n_rot + per_block - 1) / per_block;
  hipLaunchKernelGGL((swa_kernel<T, VEC>), dim3(static_cast<unsigned>(nb_copy + nb_rot)),
                     dim3(threads), 0, st, static_cast<const T*>(kv_raw), static_cast<T*>(kv_win),
                     kv_pos0, new_pos0, S_new, S_cap, D, r, make_rope_freq(r, theta), off, Gn,
                     static_cast<unsigned>(n_copy), static_cast<unsigned>(n_rot),
                     static_cast<unsigned>(nb_copy));
  return hipGetLastError();
}

hipError_t launch_swa(const void* kv_raw, void* kv_win, const int* kv_pos0, const int* new_pos0,
                      int B, int S_new, int S_cap, int D, int r, double theta, long long off,
                      int dtype, hipStream_t st) {
  const bool v8 = (D % 8 == 0);
  if (dtype == 1)
    return v8 ? swa_t<bf16_t, 8>(kv_raw, kv_win, kv_pos0, new_pos0, B, S_new, S_cap, D, r, theta, off, st)
              : swa_t<bf16_t, 2>(kv_raw, kv_win, kv_pos0, new_pos0, B, S_new, S_cap, D, r, theta, off, st);
  return v8 ? swa_t<float, 8>(kv_raw, kv_win, kv_pos0, new_pos0, B, S_new, S_cap, D, r, theta, off, st)
            : swa_t<float, 2>(kv_raw, kv_win, kv_pos0, new_pos0, B, S_new, S_cap, D, r, theta, off, st);
}

}  // namespace dsv4
