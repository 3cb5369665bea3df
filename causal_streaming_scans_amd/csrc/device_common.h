// device_common.h -- building blocks shared by the HLA kernels (gfx950 only).
//
// Every dense product in the forward path is written in one "NT" form,
//     C[i][j] += sum_k A[i][k] * Bt[j][k],
// with both operands in LDS, row-major, read contiguously along k.  A 16x16
// output tile lives in one wave as an MFMA accumulator: lane l holds rows
// 4*(l/16) + r (r = 0..3) of column l%16.
//
// bf16 tiles use V_MFMA_F32_16X16X32_BF16 (8 k-values per lane) and, for a
// trailing 16-wide k block, V_MFMA_F32_16X16X16_BF16; fp32 tiles use
// V_MFMA_F32_16X16X4_F32.  Both operands of one instruction take the same
// (lane group, slot) -> k assignment, so the sum over k is the plain dot
// product whatever order the hardware visits the k values in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hla {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
// wave index, marked wave-uniform so branches on it stay scalar
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

template <typename T> __device__ __forceinline__ float to_f(T x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x) { return static_cast<T>(x); }

// padding (in elements) that keeps every LDS row 16-byte aligned and shifts
// consecutive rows across banks
template <typename T> constexpr int pad_of() { return 16 / (int)sizeof(T); }
template <typename T> constexpr int ld_of(int cols) { return cols + pad_of<T>(); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// LDS layout of a row-major [rows][COLS] matrix of T.  bf16 matrices of 64
// columns use unpadded 128-byte rows whose eight 16-byte granules are
// permuted by XOR with sw(r) = (r & 7) ^ 5 * bit3(r) (a function of r mod
// 16, so 16-row blocks stay additive).  On gfx950's LDS (32 banks for
// writes, 64 for reads) that keeps the chunk kernels' operand-row reads,
// both transposing-read shapes and the staging stores free of bank
// conflicts, and leaves the accumulator stores at the two-way minimum of an
// 8-byte-per-lane store; a padded pitch fixes one of those at the cost of
// another.  Other matrices are padded by 16 bytes a row.
template <typename T, int COLS>
struct LdsTile {
    static constexpr bool SWZ = sizeof(T) == 2 && COLS == 64;
    static constexpr int LD = SWZ ? COLS : ld_of<T>(COLS);
    // element (r, c); c a multiple of 4 when the access is 8 or 16 bytes wide
    __device__ static __forceinline__ int off(int r, int c) {
        if constexpr (SWZ) return r * LD + ((((c >> 3) ^ (r & 7) ^ (((r >> 3) & 1) * 5)) << 3) | (c & 7));
        else return r * LD + c;
    }
};

// A plain row-major [rows][COLS] layout padded by 16 bytes a row, in the
// same form as LdsTile.
template <typename T, int COLS>
struct PadTile {
    static constexpr int LD = ld_of<T>(COLS);
    __device__ static __forceinline__ int off(int r, int c) { return r * LD + c; }
};

// ------------------------------------------ operands kept in registers
//
// MFMA shapes: a product over k uses 16x16x32 steps when k is a multiple of
// 32, else 16x16x16 throughout.  An accumulation chain never switches MFMA
// shape -- on gfx950 a 16x16x16 that takes a 16x16x32 result as its
// accumulator back to back has been seen to read it before it is final.

// MFMA operand fragments of one 16-row tile over k = 0..K, loaded once and
// reused: lane l holds row l%16 at the k offsets both operand slots use (A
// and Bt fragments are addressed alike).
template <typename T, int K> struct RowFrags;
//
// load_rows_g reads the 16 rows straight from global memory: lane l reads
// row l%16 when that row is below rows_valid and row 0 (which the caller
// guarantees to exist) otherwise, so the load is unconditional and in
// bounds; mask_rows later zeroes the rows at or past rows_valid.
template <int K> struct RowFrags<bf16, K> {
    static constexpr bool W32 = (K % 32) == 0;
    bf16x8 v8[W32 ? K / 32 : 1];
    i16x4 v4[W32 ? 1 : K / 16];
    __device__ __forceinline__ void load_rows_g(const bf16 *__restrict__ base, int ld,
                                                int rows_valid) {
        const int l = lane_id(), r = l & 15, g = l >> 4;
        const bf16 *row = base + (size_t)(r < rows_valid ? r : 0) * ld;
        if constexpr (W32) {
#pragma unroll
            for (int s = 0; s < K / 32; ++s)
                v8[s] = *reinterpret_cast<const bf16x8 *>(row + 32 * s + 8 * g);
        } else {
#pragma unroll
            for (int s = 0; s < K / 16; ++s)
                v4[s] = *reinterpret_cast<const i16x4 *>(row + 16 * s + 4 * g);
        }
    }
    __device__ __forceinline__ void mask_rows(int rows_valid) {
        if ((lane_id() & 15) >= rows_valid) {
            if constexpr (W32) {
#pragma unroll
                for (int s = 0; s < K / 32; ++s) v8[s] = bf16x8{};
            } else {
#pragma unroll
                for (int s = 0; s < K / 16; ++s) v4[s] = i16x4{};
            }
        }
    }
    // the 16-row block of an LdsTile matrix that starts at base
    template <typename TL>
    __device__ __forceinline__ void load_t(const bf16 *base) {
        const int l = lane_id(), r = l & 15, g = l >> 4;
        if constexpr (W32) {
#pragma unroll
            for (int s = 0; s < K / 32; ++s)
                v8[s] = *reinterpret_cast<const bf16x8 *>(base + TL::off(r, 32 * s + 8 * g));
        } else {
#pragma unroll
            for (int s = 0; s < K / 16; ++s)
                v4[s] = *reinterpret_cast<const i16x4 *>(base + TL::off(r, 16 * s + 4 * g));
        }
    }
};
template <int K> struct RowFrags<float, K> {
    float v[K / 4];
    __device__ __forceinline__ void load_rows_g(const float *__restrict__ base, int ld,
                                                int rows_valid) {
        const int l = lane_id(), r = l & 15, g = l >> 4;
        const float *row = base + (size_t)(r < rows_valid ? r : 0) * ld;
#pragma unroll
        for (int s = 0; s < K / 4; ++s) v[s] = row[4 * s + g];
    }
    __device__ __forceinline__ void mask_rows(int rows_valid) {
        if ((lane_id() & 15) >= rows_valid) {
#pragma unroll
            for (int s = 0; s < K / 4; ++s) v[s] = 0.f;
        }
    }
    template <typename TL>
    __device__ __forceinline__ void load_t(const float *base) {
        const int l = lane_id(), r = l & 15, g = l >> 4;
#pragma unroll
        for (int s = 0; s < K / 4; ++s) v[s] = base[TL::off(r, 4 * s + g)];
    }
};

// acc += A[0:16][0:K] * F^T with A the 16-row block of an LdsTile matrix
// that starts at A and F preloaded (F as the Bt side)
template <typename TL, int K>
__device__ __forceinline__ f32x4 mma_nt_ft(f32x4 acc, const bf16 *A, const RowFrags<bf16, K> &f) {
    const int l = lane_id(), r = l & 15, g = l >> 4;
    if constexpr (RowFrags<bf16, K>::W32) {
#pragma unroll
        for (int s = 0; s < K / 32; ++s) {
            const bf16x8 av = *reinterpret_cast<const bf16x8 *>(A + TL::off(r, 32 * s + 8 * g));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, f.v8[s], acc, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int s = 0; s < K / 16; ++s) {
            const i16x4 av = *reinterpret_cast<const i16x4 *>(A + TL::off(r, 16 * s + 4 * g));
            acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, f.v4[s], acc, 0, 0, 0);
        }
    }
    return acc;
}
template <typename TL, int K>
__device__ __forceinline__ f32x4 mma_nt_ft(f32x4 acc, const float *A, const RowFrags<float, K> &f) {
    const int l = lane_id(), r = l & 15, g = l >> 4;
#pragma unroll
    for (int s = 0; s < K / 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[TL::off(r, 4 * s + g)], f.v[s], acc, 0, 0, 0);
    return acc;
}


// Ownership of the tiles of an (nTR x nTC)-tile matrix by NW waves, in
// BR x BR blocks (BR = 2 when that still gives every wave a block).
template <int nTR, int nTC, int NW>
struct TileBlocks {
    static constexpr bool two = (nTR % 2 == 0) && (nTC % 2 == 0) && (nTR * nTC / 4 >= NW);
    static constexpr int BR = two ? 2 : 1;
    static constexpr int nBR = nTR / BR, nBC = nTC / BR, NB = nBR * nBC;
    static constexpr int PB = (NB + NW - 1) / NW;   // blocks per wave
};

// ------------------------------------------------ register-chained operands
//
// A 16x16 accumulator tile C (lane l holds C[4g + i][c], g = l/16, c = l%16)
// is, once rounded to the operand type, directly the B operand of a product
// with k running over the tile's 16 rows: lane l supplies B[k = 4g + i][c].
// The matching A operand has lane l supply A[c][4g + i] (row c, four
// consecutive k), which is also what a 16x16 accumulator of A^T holds.
// bf16: one V_MFMA_F32_16X16X16_BF16 per 16-deep step.  fp32: four
// V_MFMA_F32_16X16X4_F32, instruction m pairing slot m of every lane group
// (k = 4g + m) on both sides.  A chain of mma16 steps starts from its own
// zero accumulator and is added to any 16x16x32 partial sum with VALU adds
// (see the note on MFMA shapes above).
template <typename T> struct Frag16;
template <> struct Frag16<bf16> { i16x4 v; };
template <> struct Frag16<float> { f32x4 v; };

template <typename T> __device__ __forceinline__ Frag16<T> to_frag(f32x4 a);
template <> __device__ __forceinline__ Frag16<bf16> to_frag<bf16>(f32x4 a) {
    union { bf16 h[4]; i16x4 v; } u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u.h[i] = (bf16)a[i];
    return Frag16<bf16>{u.v};
}
template <> __device__ __forceinline__ Frag16<float> to_frag<float>(f32x4 a) { return Frag16<float>{a}; }

// value of slot i of a fragment (as the rounded operand the MFMA consumes)
__device__ __forceinline__ float frag_val(const Frag16<bf16> &f, int i) {
    union { i16x4 v; bf16 h[4]; } u;
    u.v = f.v;
    return (float)u.h[i];
}
__device__ __forceinline__ float frag_val(const Frag16<float> &f, int i) { return f.v[i]; }

__device__ __forceinline__ f32x4 mma16(f32x4 acc, Frag16<bf16> a, Frag16<bf16> b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 acc, Frag16<float> a, Frag16<float> b) {
#pragma unroll
    for (int m = 0; m < 4; ++m) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[m], b.v[m], acc, 0, 0, 0);
    return acc;
}

// Fragment whose four k-values are contiguous in LDS: lane l reads
// base[(l%16) * ld + 4g .. 4g+3].
__device__ __forceinline__ Frag16<bf16> ld_frag(const bf16 *base, int ld) {
    const int l = lane_id();
    return Frag16<bf16>{*reinterpret_cast<const i16x4 *>(base + (l & 15) * ld + ((l >> 4) << 2))};
}
__device__ __forceinline__ Frag16<float> ld_frag(const float *base, int ld) {
    const int l = lane_id();
    return Frag16<float>{*reinterpret_cast<const f32x4 *>(base + (l & 15) * ld + ((l >> 4) << 2))};
}

// ------------------------------------------------ k-major operands (gfx950)
//
// Products that contract over the row index of an LDS matrix M[k][m] (m
// contiguous) -- the token index of a row-major chunk tile -- read their
// operands with DS_READ_B64_TR_B16.  That instruction transposes within each
// 16-lane group: when lane s of group g names the 8 bytes at
// M[4g + s/4][4(s%4) .. 4(s%4)+3], lane i of the group receives M[4g + e][i]
// in slot e, i.e. the operand layout "row i, k = 4g + e" that the MFMA
// instructions take.  No transposed copy of the tile is ever stored.
typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i16x4 ds_read_tr16(const bf16 *p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(const_cast<bf16 *>(p)));
}

// Operand fragments from an LdsTile matrix M (its base) for the sub-tile whose
// first row (k) is row0 and first column col0, both multiples of 16: the
// 16-deep fragment (ld_frag_tt: slot e holds k = row0 + 4g + e) and the
// 32-deep operand of a 16x16x32 step (ld_op8_tt: slot j holds k = row0 + 8g
// + j, two transposing reads four rows apart).
template <typename TL>
__device__ __forceinline__ Frag16<bf16> ld_frag_tt(const bf16 *M, int row0, int col0) {
    const int l = lane_id(), g = l >> 4, s = l & 15;
    return Frag16<bf16>{ds_read_tr16(M + TL::off(row0 + 4 * g + (s >> 2), col0 + 4 * (s & 3)))};
}
template <typename TL>
__device__ __forceinline__ Frag16<float> ld_frag_tt(const float *M, int row0, int col0) {
    const int l = lane_id(), g = l >> 4, c = l & 15;
    f32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = M[TL::off(row0 + 4 * g + i, col0 + c)];
    return Frag16<float>{v};
}
template <typename TL>
__device__ __forceinline__ bf16x8 ld_op8_tt(const bf16 *M, int row0, int col0) {
    const int l = lane_id(), g = l >> 4, s = l & 15;
    const int r = row0 + 8 * g + (s >> 2), c = col0 + 4 * (s & 3);
    const i16x4 lo = ds_read_tr16(M + TL::off(r, c)), hi = ds_read_tr16(M + TL::off(r + 4, c));
    const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, both);
}

// Operand fragments of a column tile that is (1, 0, ..., 0) in every row:
// entry (k, m) is 1 for m = 0.  Either operand side holds m (or n) = l % 16,
// so the fragment is the same constant for both.
template <typename T> __device__ __forceinline__ Frag16<T> ones_frag();
template <> __device__ __forceinline__ Frag16<bf16> ones_frag<bf16>() {
    const short one = (lane_id() & 15) == 0 ? (short)0x3F80 : (short)0;   // bf16 1.0
    return Frag16<bf16>{i16x4{one, one, one, one}};
}
template <> __device__ __forceinline__ Frag16<float> ones_frag<float>() {
    const float one = (lane_id() & 15) == 0 ? 1.f : 0.f;
    return Frag16<float>{f32x4{one, one, one, one}};
}
__device__ __forceinline__ bf16x8 ones_op8() {
    const short one = (lane_id() & 15) == 0 ? (short)0x3F80 : (short)0;
    return __builtin_bit_cast(bf16x8, i16x8{one, one, one, one, one, one, one, one});
}

// Store four consecutive T values (one accumulator's slots, converted).
__device__ __forceinline__ void store4(bf16 *p, f32x4 a) {
    union { bf16 h[4]; uint2 v; } u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u.h[i] = (bf16)a[i];
    *reinterpret_cast<uint2 *>(p) = u.v;
}
__device__ __forceinline__ void store4(float *p, f32x4 a) { *reinterpret_cast<f32x4 *>(p) = a; }

// ------------------------------------------------------- row buffers
//
// A kernel's final output goes through a raw buffer resource over the
// segment's rows: stores past the last valid row are dropped by the
// resource's range check, so no branch per tile is needed; the chunk loads
// read through such a resource too, and read zeros past its end.  Word 3
// selects the 32-bit data format, under which untyped accesses are
// range-checked (gfx9 family).
constexpr int kBufWord3 = 0x00020000;
// Cache policy of those stores: non-temporal.  The output is written once
// and never read back by the kernel; for whole 128-byte rows this measured
// faster than the default policy (3 us of 55 per HLA-2 forward at B=8 H=16
// n=4096 d=64), while for 8-byte pieces of rows (one accumulator's slots)
// it was much slower, and non-temporal loads of q, k, v were slower too.
constexpr int kCpolNT = 2;

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(T *base, int rows, int cols) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, rows * cols * (int)sizeof(T), kBufWord3);
}

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const T *base, int rows, int cols) {
    return rows_rsrc(const_cast<T *>(base), rows, cols);
}

// 16 bytes at byte offset byte_off behind rs; zeros past the resource's end
__device__ __forceinline__ uint4 load16_buf(__amdgpu_buffer_rsrc_t rs, int byte_off) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ void store16_buf(__amdgpu_buffer_rsrc_t rs, int byte_off, uint4 x) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{x.x, x.y, x.z, x.w}, rs, byte_off, 0, kCpolNT);
}

// One accumulator's four slots (consecutive columns of one output row) at
// byte offset byte_off behind rs, with the default cache policy: a store
// past the resource's last row is dropped, so no per-lane branch is needed.
__device__ __forceinline__ void store4_rows(__amdgpu_buffer_rsrc_t rs, int byte_off, f32x4 a) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    union { bf16 h[4]; u32x2 v; } u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u.h[i] = (bf16)a[i];
    __builtin_amdgcn_raw_buffer_store_b64(u.v, rs, byte_off, 0, 0);
}
__device__ __forceinline__ void store4_rows(__amdgpu_buffer_rsrc_t rs, int byte_off, f32x4 a, float) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a), rs, byte_off, 0, 0);
}
template <typename T>
__device__ __forceinline__ void store4_row(__amdgpu_buffer_rsrc_t rs, int byte_off, f32x4 a) {
    if constexpr (sizeof(T) == 2) store4_rows(rs, byte_off, a);
    else store4_rows(rs, byte_off, a, 0.f);
}

// Write the 16 rows x COLS of a wave's LDS tile ot (layout TL) to rows
// row0 .. row0+15, columns col0 .. col0+COLS-1 of the [rows][LDG] output
// behind rs, 16 bytes a lane: each global store covers whole row pieces of
// COLS columns.  The rows were written to ot by this wave's own lanes; LDS
// operations of one wave complete in order, so no barrier.  The compiler,
// though, may not move the 16-byte reads above those writes: they are 8-byte
// stores of another type, which type-based alias analysis would let it treat
// as independent -- hence the compiler-only memory fence first.
template <typename T, typename TL, int COLS, int LDG = COLS>
__device__ __forceinline__ void store_rows_out(const T *ot, __amdgpu_buffer_rsrc_t rs, int row0,
                                               int col0 = 0) {
    __asm__ __volatile__("" ::: "memory");
    constexpr int VE = 16 / (int)sizeof(T);
    constexpr int VPR = COLS / VE;      // 16-byte pieces per row
    constexpr int NP = 16 * VPR;        // pieces of the tile
#pragma unroll
    for (int h = 0; h < (NP + kWave - 1) / kWave; ++h) {
        const int idx = h * kWave + lane_id();
        const int rr = idx / VPR, cc = (idx % VPR) * VE;
        if (NP % kWave == 0 || idx < NP) {
            const uint4 x = *reinterpret_cast<const uint4 *>(ot + TL::off(rr, cc));
            store16_buf(rs, ((row0 + rr) * LDG + col0 + cc) * (int)sizeof(T), x);
        }
    }
}

// Rows row0 .. row0+15, columns col0 .. col0+COLS-1 of an LdsTile matrix
// (tile: its base) to global rows row0g .. (row0g+15) of LDG columns through
// the buffer resource rs, in 16-byte pieces by the lanes of one wave.  The
// rows may have been written by other waves: the caller orders those writes
// before these reads with a barrier.
template <typename T, typename TL, int COLS, int LDG>
__device__ __forceinline__ void copy_rows_out(const T *tile, __amdgpu_buffer_rsrc_t rs, int row0,
                                              int row0g, int col0) {
    constexpr int VE = 16 / (int)sizeof(T);
    constexpr int VPR = COLS / VE;
    constexpr int NP = 16 * VPR;
#pragma unroll
    for (int h = 0; h < (NP + kWave - 1) / kWave; ++h) {
        const int idx = h * kWave + lane_id();
        const int rr = idx / VPR, cc = col0 + (idx % VPR) * VE;
        if (NP % kWave == 0 || idx < NP) {
            const uint4 x = *reinterpret_cast<const uint4 *>(tile + TL::off(row0 + rr, cc));
            store16_buf(rs, ((row0g + rr) * LDG + cc) * (int)sizeof(T), x);
        }
    }
}

// Row / column of accumulator element r held by this lane within its tile.
__device__ __forceinline__ int acc_row(int r) { return ((lane_id() >> 4) << 2) + r; }
__device__ __forceinline__ int acc_col() { return lane_id() & 15; }

// ------------------------------------------------------------- global loads

// 16-byte vector of T from global memory
template <typename T> struct Vec16 {
    static constexpr int N = 16 / (int)sizeof(T);
    T v[N];
};

template <typename T>
__device__ __forceinline__ Vec16<T> load16(const T *p) {
    Vec16<T> r;
    *reinterpret_cast<uint4 *>(r.v) = *reinterpret_cast<const uint4 *>(p);
    return r;
}

template <typename T>
__device__ __forceinline__ void store16(T *p, const Vec16<T> &x) {
    *reinterpret_cast<uint4 *>(p) = *reinterpret_cast<const uint4 *>(x.v);
}

// Stage `rows_valid` rows (of `ROWS`) of a [ROWS][COLS] global tile into LDS,
// row-major (dst, leading dim ldr) and/or transposed (dstT, leading dim ldt,
// dstT[c][r] = src[r][c]).  Rows >= rows_valid are written as zeros.  The
// optional transposed copy dstTw gets the value times w[r] (decay weights).
template <typename T, int ROWS, int COLS, int NT>
__device__ __forceinline__ void stage_tile(const T *__restrict__ src, int rows_valid, T *dst,
                                           int ldr, T *dstT, int ldt, T *dstTw = nullptr,
                                           const float *w = nullptr) {
    constexpr int VE = Vec16<T>::N;
    constexpr int VPR = COLS / VE;      // vectors per row
    constexpr int NV = ROWS * VPR;
    for (int idx = threadIdx.x; idx < NV; idx += NT) {
        const int r = idx / VPR, c = (idx % VPR) * VE;
        Vec16<T> x;
        if (r < rows_valid) {
            x = load16(src + (size_t)r * COLS + c);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) x.v[e] = from_f<T>(0.f);
        }
        if (dst) store16(dst + r * ldr + c, x);
        if (dstT) {
#pragma unroll
            for (int e = 0; e < VE; ++e) dstT[(c + e) * ldt + r] = x.v[e];
        }
        if (dstTw) {
            const float wr = (r < rows_valid) ? w[r] : 0.f;
#pragma unroll
            for (int e = 0; e < VE; ++e) dstTw[(c + e) * ldt + r] = from_f<T>(to_f(x.v[e]) * wr);
        }
    }
}

// Powers g^e for e = 0..count-1 into LDS, from fp64 exp2(e * log2 g) rounded
// once to fp32 (no accumulated rounding from repeated multiplication).
template <int NT>
__device__ __forceinline__ void fill_pow_table(float *tab, int count, float g) {
    const double lg = log2((double)g);
    for (int e = threadIdx.x; e < count; e += NT) tab[e] = (float)exp2(lg * (double)e);
}

__device__ __forceinline__ float pow_int(float g, long e) {
    if (e == 0 || g == 1.0f) return 1.0f;
    return (float)exp2(log2((double)g) * (double)e);
}

}  // namespace hla
