// Device helpers shared by the gfx950 kernels: storage types, 16x16 MFMA
// fragments, wave reductions, counters.
//
// Storage types: `float` (fp32 workloads) and `uint16_t` holding bf16 bit
// patterns.  Both feed the same 16x16 MFMA tile shape:
//   A fragment (16 rows x 32 k): lane l holds row l%16, k = (l/16)*8 .. +8
//   B fragment (32 k x 16 cols): lane l holds col l%16, k = (l/16)*8 .. +8
//   C (16 x 16 fp32):            lane l holds col l%16, rows (l/16)*4 .. +4
// bf16 uses one v_mfma_f32_16x16x32_bf16 per 32-k step; fp32 uses eight
// v_mfma_f32_16x16x4_f32, the i-th taking element i of every lane's 8, which
// sums over the same 32 k values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace dflash {

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per device (the attribute is per device; `done` holds one bit per device
// id below 64, larger ids set it on every launch).
inline hipError_t set_dynamic_lds_once(std::atomic<uint64_t>& done, const void* kern, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load() & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit);
  return e;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even, with gfx950's conversion instruction
// (v_cvt_pk_bf16_f32); it agrees bit for bit with the bit-level definition
// (add 0x7fff plus the kept LSB, truncate) on every non-NaN input, and maps
// NaN to NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// (a, b) -> bf16 pair, a in the low half.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <typename T> struct Store;
template <> struct Store<float> {
  static __device__ __forceinline__ float load(float v) { return v; }
  static __device__ __forceinline__ float make(float v) { return v; }
};
template <> struct Store<uint16_t> {
  static __device__ __forceinline__ float load(uint16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ uint16_t make(float v) { return f32_to_bf16(v); }
};

template <typename T> __device__ __forceinline__ float ldf(const T* p) {
  return Store<T>::load(*p);
}
template <typename T> __device__ __forceinline__ void stf(T* p, float v) {
  *p = Store<T>::make(v);
}
// Four consecutive elements, one vector access: the address must be 16-byte
// aligned for float and 8-byte aligned for bf16.
template <typename T> __device__ __forceinline__ float4 ld4(const T* p);
template <> __device__ __forceinline__ float4 ld4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <> __device__ __forceinline__ float4 ld4<uint16_t>(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
template <typename T> __device__ __forceinline__ void st4(T* p, float4 v);
template <> __device__ __forceinline__ void st4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <> __device__ __forceinline__ void st4<uint16_t>(uint16_t* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(f32x2_to_bf16x2(v.x, v.y), f32x2_to_bf16x2(v.z, v.w));
}

// Eight consecutive k values of one row.
template <typename T> struct Frag8;
template <> struct Frag8<uint16_t> { uint4 v; };
template <> struct Frag8<float> { float4 lo, hi; };

__device__ __forceinline__ void ld_frag(Frag8<uint16_t>& f, const uint16_t* p) {
  f.v = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void ld_frag(Frag8<float>& f, const float* p) {
  f.lo = *reinterpret_cast<const float4*>(p);
  f.hi = *reinterpret_cast<const float4*>(p + 4);
}
__device__ __forceinline__ void zero_frag(Frag8<uint16_t>& f) { f.v = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero_frag(Frag8<float>& f) {
  f.lo = make_float4(0.f, 0.f, 0.f, 0.f);
  f.hi = f.lo;
}

__device__ __forceinline__ f32x4 mfma16(f32x4 acc, const Frag8<uint16_t>& a,
                                        const Frag8<uint16_t>& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                 __builtin_bit_cast(bf16x8_t, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f32x4 acc, const Frag8<float>& a, const Frag8<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Wave-wide (64 lanes) reductions with a fixed butterfly order.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// (value, index) pair ordered by value, then by lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// 64-bit key whose unsigned order is (value, then lower index).
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(u) << 32) |
         static_cast<unsigned long long>(0xffffffffu - static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int argmax_key_index(unsigned long long k) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(k & 0xffffffffull));
}

// RoPE inverse frequencies theta^(-2i/d), i < d/2, formed in double on the
// host and passed by value.
struct RopeFreq {
  double inv[64];
};

// Cos/sin of the RoPE angle pos * inv: the product and its reduction to
// [-pi, pi] in double (positions reach ~10^5 radians), the sine and cosine of
// the reduced angle in float.
__device__ __forceinline__ void rope_cos_sin(int pos, double inv, float& c, float& s) {
  const double kTwoPi = 6.283185307179586476925286766559;
  const double ang = static_cast<double>(pos) * inv;
  const double r = fma(-rint(ang * (1.0 / kTwoPi)), kTwoPi, ang);
  sincosf(static_cast<float>(r), &s, &c);
}
__device__ __forceinline__ void rope_cos_sin(int pos, int i, const RopeFreq& f, float& c,
                                             float& s) {
  rope_cos_sin(pos, f.inv[i], c, s);
}

// Per-sequence bookkeeping passed by value to kernels.
constexpr int kMaxBatch = 64;
constexpr int kMaxLayers = 16;
struct SeqTable {
  int32_t len[kMaxBatch];     // committed context rows
  int32_t row0[kMaxBatch];    // first input row of the sequence (inject)
  int64_t off[kMaxBatch];     // start row of the sequence inside each head slab
  int32_t pos0[kMaxBatch];    // position of the first written row (inject)
  int32_t n;                  // sequences
  // Device-resident step: the committed lengths live in device memory (dlen,
  // clamped to [0, len_max]; len[] then holds len_max for the host's launch
  // plan), and an injection's row m is slot m % stride of sequence m / stride,
  // appended while that slot is <= dcnt[b] (accepted drafts after the anchor).
  const int32_t* dlen;
  const int32_t* dcnt;
  int32_t len_max;
  int32_t stride;
};

// Committed context rows of sequence b.
__device__ __forceinline__ int seq_len_of(const SeqTable& t, int b) {
  return t.dlen ? min(max(t.dlen[b], 0), t.len_max) : t.len[b];
}

// (max, sum of exp(x - max)) of a union of two value sets; an empty set has
// max -inf.  The log-sum-exp is max + log(sum).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  const float mx = fmaxf(m, m2);
  s = s * expf(m - mx) + s2 * expf(m2 - mx);
  m = mx;
}

// Rows of the block K/V buffer per training-layout block (a multiple of 32,
// so the V^T reads of a 32-key step stay inside the block's rows).
constexpr int kTrainSlab = 32;

// Fragment-major layout of an M x K matrix (K a multiple of 32): rows in
// groups of 16, each group stored as K/32 chunks of 16 rows x 32 columns,
// row-major inside a chunk.  The 64 lanes of one A-fragment load of the
// weight-streaming GEMM, or of one operand load of the LDS-tiled GEMM (16
// rows x 4 runs of 8 columns), then read one contiguous 1 KB chunk instead of
// 16 row pieces.  The drafter's activations use it, and so do packed weights
// (dflash_pack_weights).
__host__ __device__ __forceinline__ int64_t frag_major(int m, int k, int K) {
  return (static_cast<int64_t>(m >> 4) * (K >> 5) + (k >> 5)) * 512 + (m & 15) * 32 + (k & 31);
}

// Which sequence an input row belongs to (rows grouped by sequence).
__device__ __forceinline__ int seq_of_row(const SeqTable& t, int row) {
  int b = 0;
  for (int s = 1; s < t.n; ++s) b = (row >= t.row0[s]) ? s : b;
  return b;
}

// Input row m of an injection: its sequence b and cache position pos; false
// for a row the sequence does not append (device-resident step only).
__device__ __forceinline__ bool inject_row(const SeqTable& t, int m, int& b, int& pos) {
  if (t.dcnt) {
    b = m / t.stride;
    const int i = m - b * t.stride;
    pos = seq_len_of(t, b) + i;
    return i <= min(max(t.dcnt[b], 0), t.stride - 1);
  }
  b = seq_of_row(t, m);
  pos = t.pos0[b] + (m - t.row0[b]);
  return true;
}

}  // namespace dflash
