// LDS tile helpers shared by the bf16 MFMA kernels (gfx950 only): swizzled
// row-major tiles, transpose reads, operand packing, momentum coefficient scan.
#pragma once

#include "device_common.h"

#define TTT_LDS __attribute__((address_space(3)))
#define TTT_GLOBAL __attribute__((address_space(1)))

namespace ttt {

// Workgroup barrier that publishes the ds_write traffic issued before it.
// __syncthreads() also orders global memory (and an LDS release fence covers
// global_load_lds copies, which complete on the vector-memory counter), so
// either would make every wave wait for the next chunk's prefetch in flight.
// This one waits for the LDS counter only; the asm statements keep the
// compiler from moving memory accesses across it.  Copies made with
// global_load_lds are not covered: wait for them (vmcnt) before calling.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt not waited
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// Element offset of (row, col) in a row-major tile of W bf16 columns whose
// 16-byte chunks are permuted per row: chunk c of row r is stored at c ^ f(r).
// f is a bijection over 16 consecutive rows (so 16 lanes reading one chunk of
// 16 rows hit 16 different bank groups) whose high bits follow the row within
// a group of 4 (so the 4 rows of a transpose read, each read at up to 4
// chunks, never share a bank).  W is 64 or 128; col may point inside a chunk.
template <int W>
__device__ __forceinline__ int swz(int row, int col) {
    constexpr int NCH = W / 8;
    static_assert(NCH == 8 || NCH == 16, "tile width");
    int f;
    if constexpr (NCH == 16) {
        f = 4 * (row & 3) + ((row >> 2) & 3);
    } else {          // two rows per 64 banks
        const int h = row >> 1;
        f = 4 * (h & 1) + ((h >> 1) & 3);
    }
    return row * W + (((col >> 3) ^ f) << 3) + (col & 7);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ u32x4 lds_read16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ u32x2 lds_read8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

__device__ __forceinline__ bf16x8 join8(const u32x2& a, const u32x2& b) {
    u32x4 u = {a[0], a[1], b[0], b[1]};
    return as_bf16x8(u);
}

// Transpose read of a swizzled W-wide tile.  Lane L = 4e + q of each 16-lane
// group points at row r0 + e, columns col(q) .. col(q) + 3; lane i of the group
// receives rows r0 .. r0+3 of column col(i / 4) + i % 4.
template <int W>
__device__ __forceinline__ u32x2 tr_read(const uint16_t* tile, int r0, int col_q) {
    const int L = threadIdx.x & 15;
    const uint16_t* p = tile + swz<W>(r0 + (L >> 2), col_q);
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TTT_LDS bf16x4_t*)(p));
    return __builtin_bit_cast(u32x2, x);
}

// 8 consecutive tokens (r0 .. r0+7) as one MFMA operand; see tr_read for col_q
template <int W>
__device__ __forceinline__ u32x4 tr_read8(const uint16_t* tile, int r0, int col_q) {
    const u32x2 a = tr_read<W>(tile, r0, col_q);
    const u32x2 b = tr_read<W>(tile, r0 + 4, col_q);
    return u32x4{a[0], a[1], b[0], b[1]};
}

// scale 8 packed bf16 by 8 fp32 weights and re-round to bf16
__device__ __forceinline__ bf16x8 scale8(const u32x4& raw, const float* w) {
    u32x4 u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float lo = __uint_as_float(raw[p] << 16) * w[2 * p];
        float hi = __uint_as_float(raw[p] & 0xffff0000u) * w[2 * p + 1];
        u[p] = pack_bf16x2(lo, hi);
    }
    return as_bf16x8(u);
}

// Momentum coefficient tables by a wavefront prefix scan (one wave):
//   bp[r] = beta^r (prefix product), cc[r] = sum_{u<=r} beta^u (prefix sum), r = 0..C
template <int C>
__device__ void coefficient_scan(float beta, float* cc, float* bp) {
    const int lane = threadIdx.x & 63;
    float base_p = 1.0f, base_c = 0.0f;
    for (int r0 = 0; r0 <= C; r0 += 64) {
        float p = (lane == 0) ? 1.0f : beta;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            float o = __shfl_up(p, d, 64);
            if (lane >= d) p *= o;
        }
        float s = p;   // p = beta^lane; now the prefix sum of p
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            float o = __shfl_up(s, d, 64);
            if (lane >= d) s += o;
        }
        const int r = r0 + lane;
        if (r <= C) {
            bp[r] = base_p * p;
            cc[r] = base_c + base_p * s;
        }
        const float p63 = __shfl(p, 63, 64), s63 = __shfl(s, 63, 64);
        base_c = base_c + base_p * s63;
        base_p = base_p * p63 * beta;
    }
}

}  // namespace ttt
