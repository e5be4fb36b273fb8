// Device helpers shared by the HIP kernels of the fusion library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte staging register
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));  // 8-byte staging register

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (bf16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// 16-byte vector of T <-> floats.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const float* p, float* o) {
    float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* o) {
    *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const bf16_t* p, float* o) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* o) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(o[2 * i]) | ((uint32_t)f32_to_bf16(o[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// Two floats to packed bfloat16 (round to nearest even): low half = lo, high half = hi.  The
// casts lower to gfx950's v_cvt_pk_bf16_f32; written as casts (not inline asm) so that the
// compiler sees the instruction and inserts the wait states it needs after a transcendental
// (v_exp_f32) producing its inputs.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i
// returns element i%4 of the 8 bytes addressed by lanes i/4, i/4+4, i/4+8, i/4+12 (in that
// order): if lanes 4k..4k+3 address row k, dims 4q..4q+3 (q = lane%4) of a row-major tile,
// lane i receives column i of the 4 rows.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t lds_read_tr16(const bf16_t* p) {
  typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip; give each XCD a
// contiguous range of tile ids so that tiles sharing operands share that XCD's L2.
// Grid size must be 8 * ceil(T / 8); returns -1 for the padding workgroups.
__device__ __forceinline__ int xcd_tile(int bid, int T) {
  const int per = (T + 7) >> 3;
  const int t = (bid & 7) * per + (bid >> 3);
  return t < T ? t : -1;
}

// 16-byte buffer load of this lane's bytes [voff + soff, +16) of the buffer at `base` (nbytes
// long) straight into LDS: the wave's 64 lanes fill 1 KB at `lds` (wave-uniform), lane l at
// byte 16 l.  The descriptor, soff and lds are scalar, so a load costs no vector ALU work.
__device__ __forceinline__ void buffer_load_lds16(const void* base, int nbytes, void* lds, uint32_t voff, int soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, soff, 0, 0);
}
