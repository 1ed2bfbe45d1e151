// fa_kernel_common.h -- device-side building blocks shared by the forward
// (fa_fwd_device.h) and backward (fa_bwd_device.h) gfx950 kernels:
// vector types, constants, the MFMA dtype traits, the score-register key
// map, the LDS tile geometry with its XOR swizzle and the direct-to-LDS tile
// loader.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {


typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x2 __attribute__((__vector_size__(4)));
typedef _Float16 f16x8 __attribute__((__vector_size__(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr int kWaveRows = 32;  // query rows per wave
constexpr float kNegInf = -__builtin_inff();
// word 3 of a raw (stride 0) buffer resource on gfx9-family GPUs
constexpr int kBufferFlags = 0x00020000;
// Direct-to-LDS tile loads: the tile's buffer resource starts this many bytes
// before the tile, so that per-lane offsets stay >= 0 after the up to 3 KiB
// of immediate offset are taken out of them; and an offset that lies past
// every record count of such a resource (one tile plus kDmaBias is below
// 2^31 + 4096 bytes) or of any one-tile resource, whose loads return (or
// write) zeros.
constexpr int kDmaBias = 4096;
constexpr int kDmaPastRecords = (int)0xFFFF0000u;
// log2-domain slack before the running reference max is moved (weights <= 2^8)
constexpr float kRescaleSlack = 8.f;
// A step that skips the row max checks the weights it made instead: when one
// lane's share of a tile's weights exceeds this, the reference moves up
constexpr float kSumLimit = 256.f;

#ifndef FA_LEAD_K
#define FA_LEAD_K 3
#endif
#ifndef FA_LEAD_K_D128
#define FA_LEAD_K_D128 5
#endif
#ifndef FA_LEAD_V_D128
#define FA_LEAD_V_D128 6
#endif
#ifndef FA_LEAD_V
#define FA_LEAD_V 4
#endif

template <bool B> struct BoolTag { static constexpr bool value = B; };
template <int N> struct IntTag { static constexpr int value = N; };

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSgMfma = 0x008;
constexpr int kSgValu = 0x002 | 0x400;  // VALU including transcendental
constexpr int kSgDsRead = 0x100;

// ---------------------------------------------------------------- dtype traits
template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
    __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // two fp32 -> two RNE-rounded bf16 packed in one dword (v_cvt_pk_bf16_f32)
    __device__ static inline unsigned pack2(float x, float y) {
        bf16x2 r;
        r[0] = (__bf16)x;
        r[1] = (__bf16)y;
        return __builtin_bit_cast(unsigned, r);
    }
    // The row sum adds the fp32 weights: a sum of bf16-rounded weights is off
    // by up to 2^-8 relative on rows with few keys, which would reach LSE.
    static constexpr bool kSumRounded = false;
    __device__ static inline float sum2(unsigned, float acc) { return acc; }
};
template <> struct Mfma<_Float16> {
    __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static inline unsigned pack2(float x, float y) {
        f16x2 r;
        r[0] = (_Float16)x;
        r[1] = (_Float16)y;
        return __builtin_bit_cast(unsigned, r);
    }
    // The row sum adds the fp16-rounded weights (relative error <= 2^-11,
    // i.e. <= 4.9e-4 in LSE) two at a time: v_dot2c_f32_f16 with ones.
    static constexpr bool kSumRounded = true;
    __device__ static inline float sum2(unsigned x, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x),
                                      __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
    }
};

// max over both wave halves: permlane32_swap(x, x) returns x of the lower
// half in element 0 and x of the upper half in element 1, in every lane.
__device__ inline float halves_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key offset (within a 32-key block) of score register i in wave half hh:
// the K row fed to MFMA row m = 8*(m/8) + 4*hh' + (m%4) is chosen so that
// register i of half hh holds key 16*(i/8) + 8*hh + (i%8).
__host__ __device__ constexpr int score_key_base(int i) { return 16 * (i >> 3) + (i & 7); }
// K row fed to MFMA row m (the inverse view of the key map above).
__device__ inline int k_row_for_mfma_row(int m) {
    const int g = m >> 3, hh = (m >> 2) & 1, r = m & 3;
    return 16 * (g >> 1) + 8 * hh + 4 * (g & 1) + r;
}

// ---------------------------------------------------------------- bf16 / fp16
// K and V tiles live in LDS unpadded (rows of D elements) and are filled by
// direct-to-LDS buffer loads: each wave instruction writes 1 KiB contiguously
// (lane i -> bytes [16i, 16i+16)), so the LDS image is permuted at 16-byte
// chunk granularity instead of padded: logical chunk c of row r is stored at
// chunk c ^ swz(r).  swz makes the 16-row K operand reads and the 4-row
// transposing V reads hit distinct banks, and turns every operand address
// into (per-lane base) XOR (compile-time constant).
//
// LDS: two K stages and two V stages, one 64-key tile each.
template <int D, int NW, int BN_ = 64> struct Tile {
    static constexpr int BN = BN_;                  // keys per K/V tile (32 or 64)
    static constexpr int KB = BN / 32;              // 32-key blocks of the score MFMA
    static constexpr int NCH = BN / 16;             // 16-key chunks of the P V MFMA
    static constexpr int BM = NW * kWaveRows;       // query rows per workgroup
    static constexpr int RB = D * 2;                // bytes per LDS row
    static constexpr int MAT = BN * RB;             // bytes per K (or V) tile
    static constexpr int LDS_BYTES = 4 * MAT;  // two K and two V stages
    static constexpr int DMA_PER_WAVE = MAT / (1024 * NW);  // 1 KiB wave loads per matrix
    static_assert(DMA_PER_WAVE <= 4, "a wave's loads of a tile must fit the 12-bit immediate offset");
    static_assert(MAT % (1024 * NW) == 0, "tile must split into 1 KiB wave loads");
    static_assert(LDS_BYTES <= 65536, "LDS operand offsets must fit the 16-bit ds offset");
    // chunk permutation of row r (D = 128: 16 chunks per row; D = 64: 8;
    // D = 256: 32 chunks, two 256-byte bank lines per row, permuted within
    // each 16-chunk half as at D = 128)
    __host__ __device__ static constexpr int swz(int r) {
        if (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
        const int g = (r >> 1) & 7;
        return ((g & 1) << 2) | (g >> 1);
    }
};

// Direct-to-LDS loads of one K or V tile by one wave: load j writes the 1 KiB
// at wave_base + j KiB (lane i -> 16 bytes at +16i) from byte offset
// voff[j] + j KiB of the tile's buffer resource.  The j KiB step is the
// instruction's immediate offset, which moves both the global and the LDS
// address, so one M0 value serves all of a wave's loads of a tile.
template <int N>
__device__ inline void dma_matrix(__amdgpu_buffer_rsrc_t r, unsigned char* wave_base,
                                  const int* voff) {
    FA_LDS void* const l = (FA_LDS void*)wave_base;
    if (N > 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff[0], 0, 0, 0);
    if (N > 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff[N > 1 ? 1 : 0], 0, 1024, 0);
    if (N > 2) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff[N > 2 ? 2 : 0], 0, 2048, 0);
    if (N > 3) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, voff[N > 3 ? 3 : 0], 0, 3072, 0);
}

}  // namespace fa
