// Device helpers shared by the gfx950 kernels of the hybrid attention core.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv4 {

typedef uint16_t bf16_t;  // bf16 storage (bit pattern)

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays NaN.  gfx950 converts in hardware
// (v_cvt_pk_bf16_f32), two values per instruction.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_hw_t;

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> packed bf16 pair (low half = first).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_hw_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// N-element row chunks in the storage type <-> float registers.  N is 2, 4 or 8 and
// the address is aligned to N elements.
// ---------------------------------------------------------------------------
template <typename T>
struct Chunk;

template <>
struct Chunk<float> {
  template <int N>
  __device__ __forceinline__ static void load(const float* p, float (&v)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        float4 t = reinterpret_cast<const float4*>(p)[i];
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        float2 t = reinterpret_cast<const float2*>(p)[i];
        v[2 * i] = t.x; v[2 * i + 1] = t.y;
      }
    }
  }
  template <int N>
  __device__ __forceinline__ static void store(float* p, const float (&v)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i)
        reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < N / 2; ++i) reinterpret_cast<float2*>(p)[i] = make_float2(v[2 * i], v[2 * i + 1]);
    }
  }
};

template <>
struct Chunk<bf16_t> {
  template <int N>
  __device__ __forceinline__ static void load(const bf16_t* p, float (&v)[N]) {
    if constexpr (N == 8) {
      uint4 t = *reinterpret_cast<const uint4*>(p);
      uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else if constexpr (N == 4) {
      uint2 t = *reinterpret_cast<const uint2*>(p);
      v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xffff0000u);
      v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xffff0000u);
    } else {
      uint32_t t = *reinterpret_cast<const uint32_t*>(p);
      v[0] = __uint_as_float(t << 16); v[1] = __uint_as_float(t & 0xffff0000u);
    }
  }
  template <int N>
  __device__ __forceinline__ static void store(bf16_t* p, const float (&v)[N]) {
    if constexpr (N == 8) {
      uint4 t;
      t.x = pack_bf16x2(v[0], v[1]); t.y = pack_bf16x2(v[2], v[3]);
      t.z = pack_bf16x2(v[4], v[5]); t.w = pack_bf16x2(v[6], v[7]);
      *reinterpret_cast<uint4*>(p) = t;
    } else if constexpr (N == 4) {
      uint2 t;
      t.x = pack_bf16x2(v[0], v[1]); t.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(p) = t;
    } else {
      *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v[0], v[1]);
    }
  }
};

template <typename T>
__device__ __forceinline__ float load1(const T* p);
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load1<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

// ---------------------------------------------------------------------------
// RoPE on interleaved pairs of the trailing r channels (pair i = channels C-r+2i, C-r+2i+1,
// frequency theta^(-2i/r)).  Frequencies and angles are formed in double precision and the
// angle is reduced modulo one turn in double; the rotation is evaluated in fp32.  sin/cos of
// the reduced angle: the fp32 library functions (error ~1e-7) on the fp32 path, the hardware
// sine / cosine of the reduced turn on the bf16 path (its error is far below bf16 rounding).
// ---------------------------------------------------------------------------
constexpr int kMaxRope = 256;

// theta^(-2i/r) for i < r/2, formed on the host in double precision; kernels take it by value.
struct RopeFreq {
  double inv[kMaxRope / 2];
};

inline RopeFreq make_rope_freq(int r, double theta) {
  RopeFreq f{};
  for (int i = 0; i < r / 2 && i < kMaxRope / 2; ++i)
    f.inv[i] = pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(r));
  return f;
}

// Fill inv_freq[0 .. r/2) (one block-wide table); the caller synchronises before use.
__device__ __forceinline__ void rope_table(double* inv_freq, int r, double theta) {
  for (int i = threadIdx.x; i < r / 2; i += blockDim.x)
    inv_freq[i] = pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(r));
}

template <bool FAST = false>
__device__ __forceinline__ void rope_cs(double ang, float& c, float& s) {
  const double turns = ang * 0.15915494309189533576888376337251;  // ang / (2 pi)
  const float frac = static_cast<float>(turns - rint(turns));    // [-1/2, 1/2] turn
  if constexpr (FAST) {
    c = __builtin_amdgcn_cosf(frac);  // hardware cos / sin take turns
    s = __builtin_amdgcn_sinf(frac);
  } else {
    sincosf(frac * 6.283185307179586f, &s, &c);
  }
}

// Rotate the pairs of an N-channel chunk that starts at channel c0 (c0 even) at position pos.
template <int N, bool FAST = false>
__device__ __forceinline__ void rope_chunk(float (&v)[N], int c0, int C, int r, double pos,
                                           const double* inv_freq) {
  if (r == 0 || c0 + N <= C - r) return;
#pragma unroll
  for (int i = 0; i < N; i += 2) {
    const int ch = c0 + i;
    if (ch >= C - r) {
      float c, s;
      rope_cs<FAST>(pos * inv_freq[(ch - (C - r)) >> 1], c, s);
      const float a = v[i], b = v[i + 1];
      v[i] = a * c - b * s;
      v[i + 1] = a * s + b * c;
    }
  }
}

__host__ __device__ __forceinline__ uint32_t div_up(uint32_t a, uint32_t b) { return (a + b - 1) / b; }

// Exclusive count of `flag` over the threads before this one; *total = block-wide count.
template <int NT>
__device__ __forceinline__ int block_excl_count(bool flag, int* total, int* wave_tot) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = wave_tot[w];
    before += (w < wave) ? c : 0;
    all += c;
  }
  __syncthreads();  // wave_tot reusable
  *total = all;
  return before + in_wave;
}


}  // namespace dsv4
