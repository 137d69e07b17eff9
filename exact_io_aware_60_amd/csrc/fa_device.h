// fa_device.h -- device-side building blocks for the gfx950 attention kernels.
//
// MFMA operand layouts (v_mfma_f32_32x32x16_bf16, checked on gfx950):
//   A (32 x 16): lane l holds row l % 32, k = (l / 32) * 8 + s for slot s = 0..7
//   B (16 x 32): lane l holds col l % 32, k = (l / 32) * 8 + s
//   C (32 x 32): lane l holds col l % 32, rows (i / 4) * 8 + (l / 32) * 4 + (i % 4), i = 0..15
// The k order inside one MFMA is free as long as A and B agree, and the kernels
// use that freedom. They feed the fp32 accumulator rows of one product, in
// register order, straight into the k slots of the next product. The other
// operand is then read in the same permuted key order.
//
// LDS transpose read (ds_read_b64_tr_b16, checked on gfx950): in each 16-lane
// group, lane i supplies the address of 4 consecutive bf16 values, namely
// row (i % 16) / 4 and columns 4 * (i % 4) .. +3 of a 4 x 16 block. Lane j then
// receives column j % 16 of that block, rows 0..3. This turns a row-major
// [key][d] tile into an operand that holds consecutive keys at a fixed d.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, so that the body
// can use i in constant expressions (fully unrolled schedules).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The same product on fp16 operands (v_mfma_f32_32x32x16_f16: identical
// operand and accumulator layouts, identical rate).
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
__device__ __forceinline__ f32x16 mfma32h(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

__device__ __forceinline__ u32x4 cat(const u32x2& lo, const u32x2& hi) {
    u32x4 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = hi[0]; r[3] = hi[1];
    return r;
}

// Buffer resources and buffer -> LDS copies. A raw resource (stride 0) covers
// [base, base + bytes); loads outside it return zeros. The range check covers
// the whole offset, scalar part included (checked on MI355X: a load whose
// soffset alone passes the end returns zeros, and a wave straddling the end
// gets zeros exactly in the lanes past it), so a tile offset may be passed as
// soffset. Word 3 selects the
// 32-bit data format that raw buffer loads on gfx9-family chips expect.
// buffer_load ... lds is the MUBUF twin of global_load_lds: lane i's bytes from
// offset voff + soff land at lds_wave_base + size * i, counted by vmcnt. The
// compiler treats an in-flight global (FLAT) LDS load as a possible
// out-of-order LDS access and then waits for every outstanding LDS read
// (lgkmcnt(0)) before each use; with the buffer form its waits stay exact.
typedef __amdgpu_buffer_rsrc_t BufRes;
__device__ __forceinline__ BufRes make_bufres(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void bload_lds16(BufRes r, uint32_t voff, uint32_t soff, FA_LDS void* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void bload_lds4(BufRes r, uint32_t voff, uint32_t soff, FA_LDS void* lds_wave_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_wave_base, 4, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(0): all of this wave's vector-memory loads have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): all but the N most recently issued of this wave's
// vector-memory loads have completed (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Global 16-byte load; returns zeros when !valid (ragged tails).
__device__ __forceinline__ u32x4 gload16(const uint16_t* p, bool valid) {
    u32x4 r = {0u, 0u, 0u, 0u};
    if (valid) r = *reinterpret_cast<const u32x4*>(p);
    return r;
}

// Exchange with the lane 32 apart: returns the value held by lane l ^ 32.
__device__ __forceinline__ float swap_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    // lanes 0..31 find the partner's value in r[1], lanes 32..63 in r[0]
    return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even float -> bf16 pair packed into one dword (lo in bits 0..15).
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));  // v_cvt_pk_bf16_f32
}

// Round-to-nearest-even float -> fp16 pair packed into one dword (v_cvt_pk_f16_f32).
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    const f32x2v v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2v));
}

// Elementwise product of two packed fp16 pairs, rounded to fp16 (v_pk_mul_f16).
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, uint32_t b) {
    const f16x2v x = __builtin_bit_cast(f16x2v, a), y = __builtin_bit_cast(f16x2v, b);
    return __builtin_bit_cast(uint32_t, x * y);
}

// ---- padded LDS tiles ----
// A padded tile stores row r of a [rows x D] 16-bit tile at byte r * STRIDE, so
// every fragment address is (lane base) + (compile-time offset): no per-read
// swizzle arithmetic. The padding is chosen for the read pattern:
//  * row tiles (16-byte reads, 16 lanes = 16 consecutive rows at one column):
//    STRIDE = 2D + 16, so the 16 rows start 16 bytes apart modulo the 256-byte
//    bank line and hit distinct banks;
//  * transposed tiles (ds_read_b64_tr_b16: 32 lanes read 4 consecutive rows x
//    64 bytes): STRIDE = 2D + 64 (2D is 128 or 256), so the 4 rows land on
//    distinct 64-byte quarters of the bank line.
template <int D> struct RowPad { static constexpr int STRIDE = 2 * D + 16; };
template <int D> struct TrPad { static constexpr int STRIDE = 2 * D + 64; };

// Bytes a padded tile of ROWS rows occupies, rounded up to whole 1 KiB blocks
// (the unit one wave's global->LDS copy writes).
template <int STRIDE, int ROWS>
constexpr int padded_tile_bytes() { return (ROWS * STRIDE + 1023) / 1024 * 1024; }

// Copy of a padded tile through a buffer resource, with each lane's source
// offsets computed once. Source row r of the tile starts `pitch` elements
// after row r - 1 and holds ELEMS 16-bit values; the tile has ROWS rows of
// STRIDE bytes. Rows past the resource's end read as zeros. Every wave issues
// exactly NT loads per copy (a wave with no block left re-copies the tile's
// last block: the same bytes to the same place).
template <int ELEMS, int STRIDE, int ROWS, int NW>
struct CopyPlan {
    static constexpr int SPR = STRIDE / 16;
    static constexpr int NB = padded_tile_bytes<STRIDE, ROWS>() / 1024;
    static constexpr int NT = (NB + NW - 1) / NW;
    uint32_t off[NT];   // byte offset of this lane's 16 bytes of block min(w + NW*t, NB - 1)

    __device__ __forceinline__ void init(int w, int lane, int pitch) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int u = w + NW * t < NB ? w + NW * t : NB - 1;
            const int slot = u * 64 + lane;
            int row = slot / SPR, c = slot - (slot / SPR) * SPR;
            if (c >= ELEMS / 8 || row >= ROWS) {   // padding slot: any in-tile source
                c = 0;
                row = row < ROWS ? row : ROWS - 1;
            }
            off[t] = (uint32_t)(row * pitch + c * 8) * 2u;
        }
    }
    // Block t of wave ws (a scalar wave index).
    __device__ __forceinline__ void copy_one(int t, BufRes r, uint32_t soff, FA_LDS uint8_t* __restrict__ tile,
                                             int ws) const {
        const int u = ws + NW * t < NB ? ws + NW * t : NB - 1;
        bload_lds16(r, off[t], soff, tile + u * 1024);
    }
    // soff: byte offset of the tile's first row in the resource (uniform);
    // w: the wave index. It is made scalar here, at the copy, rather than once
    // per kernel: a scalar wave index held across the whole kernel has been
    // seen to make the register allocator copy accumulators around.
    __device__ __forceinline__ void copy(BufRes r, uint32_t soff, FA_LDS uint8_t* __restrict__ tile,
                                         int w) const {
        const int ws = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
        for (int t = 0; t < NT; ++t) copy_one(t, r, soff, tile, ws);
    }
};

// ---- swizzled LDS tiles ----
// A swizzled tile stores a [ROWS x L bytes] 16-bit tile densely (row r at byte
// r * L) and puts 16-byte chunk c of row r at chunk position c ^ key(r):
//   L = 512 (32 chunks): key(r) = r & 15 (two bank lines per row: chunk c sits
//                        in bank group c % 16 of its line whatever the row, so
//                        the key alone spreads 16 rows over the 16 groups);
//   L = 256 (16 chunks): key(r) = r & 15;
//   L = 128 (8 chunks):  key(r) = (r >> 1) & 7.
// A 16-byte row read in which 16 lanes take 16 consecutive rows (starting at a
// multiple of 16) at one logical chunk then touches 16 distinct 16-byte bank
// groups: with L = 256 the positions differ, with L = 128 rows of one parity
// do and the parities fill the two halves of the 256-byte bank line. (Measured
// on MI355X with the MFMA operand lane pattern, row l32 and half hh: both
// layouts read at 223-230 B/clk per CU, as fast as the padded rows.) Unlike
// padding, the tile is whole 1 KiB blocks of data only, so a copy moves no pad
// bytes and splits evenly over 4 or 8 waves.
template <int L>
__host__ __device__ constexpr int swz_key(int r) {
    static_assert(L == 512 || L == 256 || L == 128, "swizzled rows are 128, 256 or 512 bytes");
    return L >= 256 ? (r & 15) : ((r >> 1) & 7);
}

// The same for tiles read with ds_read_b64_tr_b16, where 32 lanes read 4
// consecutive rows (starting at a multiple of 4) x 64 bytes at one column: the
// 64-byte quarters of a row are permuted instead, quarter q of row r stored at
// quarter q ^ tr_key(r), so the 4 rows land on the 4 distinct 64-byte quarters
// of the 256-byte bank line (L = 512 likewise: quarter q of any row is in
// quarter q % 4 of its line; L = 128: two rows share a line, and the key
// separates the rows of one parity). In 16-byte chunk units the key is
// tr_key(r) << 2.
template <int L>
__host__ __device__ constexpr int tr_key(int r) {
    static_assert(L == 512 || L == 256 || L == 128, "swizzled rows are 128, 256 or 512 bytes");
    return L >= 256 ? (r & 3) : ((r >> 1) & 1);
}
template <int L> struct RowKey { __host__ __device__ static constexpr int key(int r) { return swz_key<L>(r); } };
template <int L> struct TrKey { __host__ __device__ static constexpr int key(int r) { return tr_key<L>(r) << 2; } };

// Copy of a swizzled [ROWS x L] tile through a buffer resource: wave w copies
// 1 KiB blocks w, w + NW, ... (NT of them, the same count on every wave).
// 16-byte chunk c of row r goes to chunk position c ^ Key::key(r). Source row
// r starts `pitch` elements after row r - 1; rows past the resource's end read
// as zeros. Each lane's source offsets are computed once.
//
// PAD: the source rows hold only the first `dr` (a multiple of 8, < L / 2)
// 16-bit values of each tile row. Lanes whose chunk lies past them issue no
// load, so their LDS bytes keep what the kernel put there (zeros; see
// lds_zero): a tile row is then the source row followed by zero columns.
template <int L, int ROWS, int NW, class Key = RowKey<L>, bool PAD = false>
struct CopyPlanSwz {
    static constexpr int NB = ROWS * L / 1024;
    static constexpr int NT = NB / NW;
    static_assert(NB % NW == 0, "the tile splits evenly over the waves");
    static_assert(NT <= 32, "one mask bit per block");
    uint32_t off[NT];
    uint32_t vmask;   // PAD: bit t set when block t's chunk of this lane is a source chunk
    __device__ __forceinline__ void init(int w, int lane, int pitch, int dr = 0) {
        vmask = 0;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int pos = (w + NW * t) * 1024 + lane * 16;
            const int row = pos / L, phys = (pos % L) / 16;
            const int c = phys ^ Key::key(row);
            off[t] = (uint32_t)(row * pitch + c * 8) * 2u;
            if (PAD && c * 8 < dr) vmask |= 1u << t;
        }
    }
    // Block t of wave ws (a scalar wave index).
    __device__ __forceinline__ void copy_one(int t, BufRes r, uint32_t soff, FA_LDS uint8_t* __restrict__ tile,
                                             int ws) const {
        if (!PAD || ((vmask >> t) & 1u)) bload_lds16(r, off[t], soff, tile + (ws + NW * t) * 1024);
    }
    __device__ __forceinline__ void copy(BufRes r, uint32_t soff, FA_LDS uint8_t* __restrict__ tile, int w) const {
        const int ws = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
        for (int t = 0; t < NT; ++t) copy_one(t, r, soff, tile, ws);
    }
};

// Zero `bytes` bytes of LDS from `base` (a multiple of 16 bytes), all threads
// of the workgroup taking part; the caller synchronises before the bytes are
// written again by global->LDS copies.
__device__ __forceinline__ void lds_zero(FA_LDS uint8_t* base, int bytes, int tid, int nthreads) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < bytes; o += nthreads * 16) *reinterpret_cast<FA_LDS u32x4*>(base + o) = z;
}

// ---- per-lane fragment reads ----
// Both structs read the A-operand fragment of a 32-row block: chunk pair c
// (16-bit elements c*16 + hh*8 ..) of row R0 + l32, R0 a multiple of 32 known
// at compile time. They share one interface, so a kernel can take either
// layout for a tile.

// Padded rows, STRIDE bytes apart.
template <int STRIDE>
struct PadRows {
    int b0;
    __device__ __forceinline__ void init(int l32, int hh) { b0 = l32 * STRIDE + hh * 16; }
    __device__ __forceinline__ u32x4 read(const FA_LDS uint8_t* tile, int R0, int c) const {
        return *reinterpret_cast<const FA_LDS u32x4*>(tile + b0 + R0 * STRIDE + c * 32);
    }
};

// L-byte rows swizzled with swz_key<L>, from one register per lane: the pair
// sits at b0 ^ (c << 5), plus R0 * L (key bit 0 flips the half, the higher key
// bits the pair index; R0 leaves the key unchanged). The XOR is applied to the
// whole LDS address, so the tile must start on an L-byte boundary. With PIN it
// is an asm statement at each read, which the compiler may not hoist out of a
// loop, so the offsets do not hold one register each; R0 * L folds into the
// read's offset field.
template <int L, bool PIN = true>
struct SwzRowRead {
    int b0;
    __device__ __forceinline__ void init(int l32, int hh) {
        const int key = swz_key<L>(l32);
        b0 = l32 * L + ((hh ^ (key & 1)) << 4) + ((key >> 1) << 5);
    }
    __device__ __forceinline__ u32x4 read(const FA_LDS uint8_t* tile, int R0, int c) const {
        const uint32_t a = (uint32_t)(uintptr_t)tile + (uint32_t)b0;
        uint32_t x = a ^ (uint32_t)(c << 5);
        if constexpr (PIN)
            if (c != 0) asm volatile("v_xor_b32 %0, %1, %2" : "=v"(x) : "i"(c << 5), "v"(a));
        return *reinterpret_cast<const FA_LDS u32x4*>((const FA_LDS uint8_t*)(uintptr_t)x + R0 * L);
    }
};
using Swz128 = SwzRowRead<128>;

// 16-byte and transposed 8-byte reads at a byte offset into a padded tile.
__device__ __forceinline__ u32x4 lds_read16b(const FA_LDS uint8_t* base, int byte_off) {
    return *reinterpret_cast<const FA_LDS u32x4*>(base + byte_off);
}
__device__ __forceinline__ u32x2 lds_read_trb(const FA_LDS uint8_t* base, int byte_off) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<FA_LDS s16x4*>(const_cast<FA_LDS uint8_t*>(base + byte_off)));
    return __builtin_bit_cast(u32x2, r);
}

}  // namespace fa
