// sg_device.h -- device helpers shared by the gfx950 kernels of libskinny_gemm.
//
// Data conventions: bf16 values are raw 16-bit patterns; 8 of them travel as
// one uint4 (a 16-byte global load).  All accumulation is fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sg {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kBlock = 256;          // threads per workgroup (4 waves)
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kPiece = 8;            // bf16 elements per 16-byte load
constexpr int kLaneSpan = kWave * kPiece;  // 512 elements: one 16-byte load per lane

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Index of the calling wavefront inside its workgroup, as a wave-uniform
// (scalar) value: the compiler cannot prove threadIdx.x / 64 is uniform, and
// anything derived from a value it thinks divergent (buffer descriptors,
// row indices) would otherwise be handled lane by lane.
__device__ __forceinline__ int wave_id_in_block() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Raw buffer resource over [base, base + bytes): a 16-byte load at a byte
// offset >= bytes returns zeros in hardware instead of touching memory, so
// ragged tails need no per-lane branches.  Word 3 = 0x00020000 is the gfx9
// family (gfx950 included) raw-buffer format: 32-bit data, no swizzle.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Cache policy of a load: kCached for data other waves reuse (activations),
// kStream (the non-temporal bit) for weights each call reads exactly once.
// Measured on MI355X: a 117 MB weight stream runs about 8% faster with the
// non-temporal hint.
constexpr int kCached = 0;
constexpr int kStream = 2;

template <int POLICY = kCached>
__device__ __forceinline__ uint4 load16(rsrc_t r, uint32_t byte_offset) {
    return __builtin_bit_cast(uint4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, POLICY));
}

// Sum of the 8 products a[i]*b[i] of two bf16x8 vectors, added to acc.
// v_dot2c_f32_bf16 multiplies bf16 pairs exactly and accumulates in fp32.
__device__ __forceinline__ float dot8(const uint4 a, const uint4 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                          __builtin_bit_cast(bf16x2_t, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                          __builtin_bit_cast(bf16x2_t, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                          __builtin_bit_cast(bf16x2_t, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                          __builtin_bit_cast(bf16x2_t, b.w), acc, false);
    return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes of a wavefront; every lane receives the total.
// Within each 16-lane row: DPP quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror (each step adds the partner lane's partial).
// Across rows: the four row totals are read from lanes 0/16/32/48.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// Sum of v over the 16 lanes of its DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    return v;
}

// Reduce-scatter of V values (V % 4 == 0) over the 64 lanes of a wave.
// Returns, in lane q*16 + i (i < V/4), the wave-wide sum of value
// q*V/4 + i; other lanes return a value of no meaning.
template <int V>
__device__ __forceinline__ float reduce_scatter(const float (&a)[V], int lane) {
    static_assert(V % 4 == 0, "pad V to a multiple of 4");
    static_assert(V <= 4 * 16, "at most 16 values per 16-lane row");
    constexpr int H = V / 2, Q = V / 4;
    float b[H];
#pragma unroll
    for (int j = 0; j < H; ++j) {
        // lanes 0-31 keep value j summed over lanes l and l+32, lanes 32-63 value j+H
        const auto p = __builtin_amdgcn_permlane32_swap(as_u(a[j]), as_u(a[j + H]), false, false);
        b[j] = as_f(p[0]) + as_f(p[1]);
    }
    float c[Q];
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        // rows 0 and 2 keep b[j], rows 1 and 3 keep b[j+Q], each summed over a row pair
        const auto p = __builtin_amdgcn_permlane16_swap(as_u(b[j]), as_u(b[j + Q]), false, false);
        c[j] = row16_sum(as_f(p[0]) + as_f(p[1]));
    }
    const int i = lane & 15;
    float out = c[0];
#pragma unroll
    for (int j = 1; j < Q; ++j) out = (i == j) ? c[j] : out;
    return out;
}

// Value index held by a lane after reduce_scatter<V>, or -1.
template <int V>
__device__ __forceinline__ int scatter_index(int lane) {
    constexpr int Q = V / 4;
    const int i = lane & 15;
    return i < Q ? (lane >> 4) * Q + i : -1;
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Where a finished output element goes.  Either a split-K partial slot, or
// the final epilogue: value = acc (+ r[i] when a residual is given), stored
// as fp32 and/or bf16 (RNE of the fp32 value).
struct Epilogue {
    float* partial;         // split partials when split_k > 1 ([S, M, N] from the vector-ALU
                            // kernel, [S, N, 16*ceil(M/16)] from the chunk kernel), else nullptr
    float* y_f32;           // nullable
    uint16_t* y_bf16;       // nullable; may equal r (in place)
    const uint16_t* r;      // residual [M, N] or nullptr
};

__device__ __forceinline__ void store_final(const Epilogue& ep, int64_t i, float acc) {
    float v = acc;
    if (ep.r) v += bf16_to_f32(ep.r[i]);
    if (ep.y_f32) ep.y_f32[i] = v;
    if (ep.y_bf16) ep.y_bf16[i] = f32_to_bf16(v);
}

}  // namespace sg
