// Quantization (the encoder): fp32 / bf16 / f16 matrix -> packed ROCmFP4 rows.
//
// "Feasibility Report: Porting ROCmFP4 to Atlas", "What is ROCmFP4?", defines the
// decoder (Block Layout, Codebook10 Value Table, Scale Format) and motivates the
// codebook's top magnitude of 10 (retuned down from 12 to limit the pull of outliers),
// which presumes an encoder that sends a group's largest magnitude to code 10. It
// prints no encoder; this one is the plainest the decoder supports:
//   * scale byte: per scale group (16 weights dual, 32 fast) the smallest b in 0..126
//     whose decoded scale S(b) has 10 * S(b) >= max |w|; b = 126 when none has
//     (saturation; the non-finite byte 127 is never written);
//   * index: the codebook entry nearest to w / S(b), ties to the smaller magnitude;
//     zero magnitude is always index 0 (never the second zero, index 8).
// Every decision is an exact comparison in fp32: S(b) has at most four significant
// bits and so have 10 and the midpoints between codebook magnitudes (0.5, 1.5, 2.5,
// 3.5, 5, 7, 9), so 10 * S(b) and midpoint * S(b) are exact, and every input value is
// exact in fp32. Non-finite inputs: a NaN or infinity makes its group saturate
// (b = 126); NaN weights get index 0, infinities +-10.
//
// Mapping. Four consecutive threads own one block; thread s reads weights 8s .. 8s+7
// (one 16-byte load for 16-bit inputs, two for fp32), so a wavefront reads contiguous
// memory. Group maxima are combined over the two (dual) or four (fast) threads of a
// group with lane shuffles, and the threads holding weights t and t + 16 meet through
// a shuffle to form the qs bytes (t in the low nibble, t + 16 in the high one). A
// workgroup packs kSeg blocks into LDS and writes that output segment, a multiple of
// 16 bytes, with 16-byte stores; the final segment of the matrix ends with byte stores.
// Output rows are back to back, so the output is one contiguous byte range.

#include "rfp4_decode.h"
#include "rfp4_internal.h"

namespace rfp4 {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kPasses = 4;                              // blocks per 4-thread team
constexpr int kSeg = kQuantThreads / 4 * kPasses;       // blocks per workgroup segment
constexpr int kMaxSegBytes = kSeg * 18;

// Scale of a group: the smallest b in 0..126 whose decoded scale S(b) has
// 10 * S(b) >= amax, with amax given by its fp32 bit pattern (NaN patterns compare
// above every finite value and infinity, so they saturate at b = 126).
// r = fl(fl(0.1 * amax) * (1 - 2^-20)) is at most amax / 10 and within a relative
// 2^-19 of it, far closer than the relative spacing of the decoded scales (>= 1/16),
// so the smallest decoded scale >= r is the answer or the one below it, and one exact
// comparison settles which. Decoded scales below 2^-7 are b * 2^-10; from 2^-7 up
// they are the fp32 values with three mantissa bits, whose bit patterns give b
// directly (fp32 exponent bias 127 against 7 + 1 for the halved E4M3 value).
struct GroupScale {
  float s;     // S(b)
  uint32_t b;  // scale byte
};

__device__ __forceinline__ GroupScale group_scale(uint32_t amax_bits) {
  constexpr uint32_t kReach126 = 0x450C0000u;  // bits of 10 * S(126) = 2240
  const float q = __uint_as_float(amax_bits);
  const float r = (q * 0.1f) * (1.0f - 0x1p-20f);
  const bool small = r < 0x1p-7f;
  const float s_small = __builtin_ceilf(r * 1024.0f) * 0x1p-10f;
  const float s_large = __uint_as_float((__float_as_uint(r) + 0xFFFFFu) & 0xFFF00000u);
  float s = small ? s_small : s_large;
  const float step = small ? 0x1p-10f : __uint_as_float(__float_as_uint(s) & 0x7F800000u) * 0.125f;
  s = (10.0f * s < q) ? s + step : s;
  uint32_t b = s < 0x1p-7f ? static_cast<uint32_t>(s * 1024.0f) : (__float_as_uint(s) >> 20) - 952u;
  if (amax_bits > kReach126) {
    s = 224.0f;
    b = 126;
  }
  return {s, b};
}

// Keeps a value in a register as computed (stops the compiler from rewriting a
// select between two products as a product of a select, which costs a multiply per
// weight).
__device__ __forceinline__ float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Lane exchange inside groups of four lanes (DPP quad permutations).
template <int XOR>
__device__ __forceinline__ uint32_t quad_xor(uint32_t v) {
  constexpr int ctrl = XOR == 1 ? 0xB1 : 0x4E;  // [1,0,3,2] and [2,3,0,1]
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), ctrl, 0xF, 0xF, false));
}

// Eight consecutive source values of one thread: raw words plus helpers.
template <int DT>
struct Eight {
  uint32_t d[DT == kF32 ? 8 : 4];

  __device__ __forceinline__ float value(int i) const {
    if constexpr (DT == kF32) return __uint_as_float(d[i]);
    else if constexpr (DT == kBF16)
      return __uint_as_float((i & 1) ? (d[i >> 1] & 0xFFFF0000u) : (d[i >> 1] << 16));
    else
      return static_cast<float>(
          __builtin_bit_cast(_Float16, static_cast<uint16_t>(d[i >> 1] >> (16 * (i & 1)))));
  }

  // Largest magnitude as an fp32 bit pattern (integer maximum of the magnitude bits,
  // which orders non-negative values and puts NaN above infinity).
  __device__ __forceinline__ uint32_t amax_bits() const {
    if constexpr (DT == kF32) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, d[i] & 0x7FFFFFFFu);
      return m;
    } else {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo = max(lo, d[i] & 0x7FFFu);
        hi = max(hi, (d[i] >> 16) & 0x7FFFu);
      }
      const uint32_t m = max(lo, hi);
      if constexpr (DT == kBF16) return m << 16;
      return __float_as_uint(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(m))));
    }
  }

  // Sign bits of values 4h .. 4h+3 at bit 7 of bytes 0..3.
  __device__ __forceinline__ uint32_t signs(int h) const {
    if constexpr (DT == kF32) {
      const uint32_t a = __builtin_amdgcn_perm(d[4 * h + 1], d[4 * h], 0x0C0C0703u);
      const uint32_t b = __builtin_amdgcn_perm(d[4 * h + 3], d[4 * h + 2], 0x07030C0Cu);
      return a | b;
    } else {
      return __builtin_amdgcn_perm(d[2 * h + 1], d[2 * h], 0x07050301u);
    }
  }
};

template <int LAYOUT, int DT>
__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const uint8_t* __restrict__ src,
                                                              int64_t lds_bytes, int64_t nb,
                                                              int64_t total_blocks,
                                                              int64_t segments,
                                                              uint8_t* __restrict__ out) {
  constexpr int BB = block_bytes(LAYOUT);
  constexpr int ESIZE = DT == kF32 ? 4 : 2;
  constexpr int WORDS = DT == kF32 ? 8 : 4;
  __shared__ __attribute__((aligned(16))) uint8_t seg_buf[kMaxSegBytes];

  const int tid = threadIdx.x;
  const int s = tid & 3;      // thread within its block's team
  const int team = tid >> 2;  // 0 .. 63
  const uint32_t nb32 = static_cast<uint32_t>(nb);  // nb < 2^26

  for (int64_t seg = blockIdx.x; seg < segments; seg += gridDim.x) {
    const int64_t first = seg * kSeg;
    const int64_t row_f = first / nb;  // uniform over the workgroup
    const uint32_t j_f = static_cast<uint32_t>(first - row_f * nb);

    Eight<DT> v[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
#pragma unroll
      for (int i = 0; i < WORDS; ++i) v[p].d[i] = 0;
      if (first + team + 64 * p < total_blocks) {
        // Block column j_f + team + 64p (< nb + 256) split into row and column.
        uint32_t jj = j_f + team + 64u * p;
        int64_t row = row_f;
        if (nb32 >= 256) {  // at most one wrap
          const bool wrap = jj >= nb32;
          jj -= wrap ? nb32 : 0u;
          row += wrap;
        } else {
          row += jj / nb32;
          jj %= nb32;
        }
        const uint8_t* q = src + row * lds_bytes + (static_cast<int64_t>(jj) * 32 + 8 * s) * ESIZE;
        const uint4 a = *reinterpret_cast<const uint4*>(q);
        v[p].d[0] = a.x; v[p].d[1] = a.y; v[p].d[2] = a.z; v[p].d[3] = a.w;
        if constexpr (DT == kF32) {
          const uint4 b = *reinterpret_cast<const uint4*>(q + 16);
          v[p].d[4] = b.x; v[p].d[5] = b.y; v[p].d[6] = b.z; v[p].d[7] = b.w;
        }
      }
    }

#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      uint32_t amax = v[p].amax_bits();
      amax = max(amax, quad_xor<1>(amax));
      if constexpr (LAYOUT == kFast) amax = max(amax, quad_xor<2>(amax));
      const GroupScale g = group_scale(amax);
      const uint32_t b = g.b;
      // Midpoints between consecutive codebook magnitudes, times the scale (exact).
      const float t0 = opaque(0.5f * g.s), t1 = opaque(1.5f * g.s), t2 = opaque(2.5f * g.s);
      const float t3 = opaque(3.5f * g.s), t4 = opaque(5.0f * g.s), t5 = opaque(7.0f * g.s);
      const float t6 = opaque(9.0f * g.s);
      uint32_t codes[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t mag = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // Number of midpoints below |w| by a three-level search; every comparison
          // with NaN is false, so NaN gets magnitude 0.
          const float a = __builtin_fabsf(v[p].value(4 * h + i));
          const bool c1 = a > t3;
          const bool c2 = a > (c1 ? t5 : t1);
          const bool c3 = a > (c1 ? (c2 ? t6 : t4) : (c2 ? t2 : t0));
          mag |= ((c1 ? 4u : 0u) | (c2 ? 2u : 0u) | (c3 ? 1u : 0u)) << (8 * i);
        }
        // Sign (index bit 3) only where the magnitude is non-zero: bytes are <= 7, so
        // adding 7 sets bit 3 exactly for the non-zero ones.
        const uint32_t nonzero = (mag + 0x07070707u) & 0x08080808u;
        codes[h] = mag | ((v[p].signs(h) >> 4) & nonzero);
      }
      // Threads 0, 1 hold weights 0..15 (low nibbles), threads 2, 3 weights 16..31.
      const uint32_t hi0 = quad_xor<2>(codes[0]);
      const uint32_t hi1 = quad_xor<2>(codes[1]);
      if (first + team + 64 * p < total_blocks) {
        uint8_t* d = seg_buf + (64 * p + team) * BB;
        if (s < 2) {
          const uint32_t q0 = codes[0] | (hi0 << 4);
          const uint32_t q1 = codes[1] | (hi1 << 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            d[8 * s + i] = static_cast<uint8_t>(q0 >> (8 * i));
            d[8 * s + 4 + i] = static_cast<uint8_t>(q1 >> (8 * i));
          }
        }
        if (s == 0) d[16] = static_cast<uint8_t>(b);
        if (LAYOUT == kDual && s == 2) d[17] = static_cast<uint8_t>(b);
      }
    }
    __syncthreads();

    const int64_t nblk = min(static_cast<int64_t>(kSeg), total_blocks - first);
    const int bytes = static_cast<int>(nblk) * BB;
    uint8_t* o = out + first * BB;  // 16-byte aligned: kSeg * BB is a multiple of 16
    typedef uint32_t ntu4 __attribute__((ext_vector_type(4)));
    for (int c = tid; c < bytes / 16; c += kQuantThreads)  // written once: non-temporal
      __builtin_nontemporal_store(*reinterpret_cast<const ntu4*>(seg_buf + 16 * c),
                                  reinterpret_cast<ntu4*>(o + 16 * c));
    const int tail = bytes & 15;
    if (tid < tail) o[bytes - tail + tid] = seg_buf[bytes - tail + tid];
    __syncthreads();
  }
}

static_assert((kSeg * 18) % 16 == 0 && (kSeg * 17) % 16 == 0, "segments end on 16 bytes");

template <int LAYOUT>
hipError_t launch_layout(const void* src, int dtype, int64_t lds, int64_t nb, int64_t total,
                         uint8_t* out, hipStream_t stream) {
  const int64_t segments = (total + kSeg - 1) / kSeg;
  const unsigned grid = static_cast<unsigned>(min(segments, static_cast<int64_t>(1) << 20));
  const uint8_t* p = static_cast<const uint8_t*>(src);
  if (dtype == kF32)
    quant_kernel<LAYOUT, kF32><<<grid, kQuantThreads, 0, stream>>>(p, lds * 4, nb, total, segments, out);
  else if (dtype == kBF16)
    quant_kernel<LAYOUT, kBF16><<<grid, kQuantThreads, 0, stream>>>(p, lds * 2, nb, total, segments, out);
  else
    quant_kernel<LAYOUT, kF16><<<grid, kQuantThreads, 0, stream>>>(p, lds * 2, nb, total, segments, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void* src, int dtype, int64_t n, int64_t k, int64_t lds,
                           int layout, uint8_t* out, hipStream_t stream) {
  const int64_t nb = k / 32;
  const int64_t total = n * nb;
  return layout == kDual ? launch_layout<kDual>(src, dtype, lds, nb, total, out, stream)
                         : launch_layout<kFast>(src, dtype, lds, nb, total, out, stream);
}

}  // namespace rfp4
