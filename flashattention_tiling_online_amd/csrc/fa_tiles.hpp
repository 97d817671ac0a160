// fa_tiles.hpp — operand tiles shared by the gfx950 attention kernels.
//
// The kernels contract 32x32 blocks on v_mfma_f32_32x32x16_{bf16,f16}.  An A operand
// comes from LDS, B from registers:
//   * row tiles: a [64, D] block of a [rows, D] matrix (K, V, Q or dO) with padded
//     rows; lane (row = lane % 32, half h) reads elements 16c + 8h .. +8 of its row
//     with one ds_read_b128 — the A operand of a product that contracts over D
//     (S = Q K^T, dP = dO V^T and their transposes);
//   * the same row tiles read transposed (tr_operand): the A operand of a product
//     that contracts over the tile's rows (O^T += V^T P^T, dV^T += dO^T P,
//     dK^T += Q^T dS, dQ^T += K^T dS^T), its k-slots in the order a 32x32 accumulator
//     holds them in registers, so that the accumulator rounded to T is the matching B
//     operand as it stands;
//   * transposed tiles (the d = 64 forward): D rows of 64 entries (144-byte stride),
//     written from registers in that same order (slots 16c + 8h + 0..3 hold entries
//     16c + 4h + 0..3, slots 16c + 8h + 4..7 hold 16c + 8 + 4h + 0..3);
//   * loads go through buffer resources bounded by the head's rows, so rows past the
//     end read as zero.
#pragma once

#include "fa_common.hpp"

namespace fa {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

template <typename T>
struct Mfma16;

template <>
struct Mfma16<__bf16> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // acc + (sum of the two elements of a packed pair), fp32 accumulate
    static __device__ __forceinline__ float dot_ones(uint32_t pair, float acc)
    {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
    }
};

template <>
struct Mfma16<_Float16> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float dot_ones(uint32_t pair, float acc)
    {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
    }
};

// Records of a buffer resource are capped at kRsrcCap bytes: every access through
// one lies within 128 rows of its base (at most 64 KB), and the cap keeps the byte
// count inside 32 bits for any head.  kDmaSkip is beyond every resource's records.
constexpr int kRsrcCap = 1 << 30;
constexpr int kDmaSkip = 0x7FFFFFF0;

// Byte offset, inside a tile of the [rows, D] matrix in memory, that lane `lane` of
// the 1-KB DMA block `blk` fetches for an LDS tile with row stride `str`: the LDS
// byte it lands on is blk*1024 + 16*lane.  kDmaSkip for lanes that land on row
// padding: out of range, they read zero (and write it into the padding, which is
// never read), so every lane of a block issues the same instruction unmasked.
template <int D>
__device__ __forceinline__ int dma_src(int blk, int lane, int str)
{
    const int pos = blk * 1024 + 16 * lane;
    const int row = pos / str;
    const int ch = (pos - row * str) / 16;
    return ch < (2 * D) / 16 ? row * (2 * D) + ch * 16 : kDmaSkip;
}

// Word 3 of a gfx9 buffer resource for untyped (raw) loads: 32-bit data format.
constexpr int kRsrcWord3 = 0x00020000;

// Buffer resource over rows [row0, nrows) of a [nrows, D] matrix: offsets past the
// end (or past kRsrcCap) read as zero.
template <int D, typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const T* base, int row0, int nrows)
{
    const int64_t n = nrows > row0 ? nrows - row0 : 0;
    const int64_t bytes = n * D * (int64_t)sizeof(T);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base) + (size_t)row0 * D, 0,
                                             bytes < kRsrcCap ? (int)bytes : kRsrcCap,
                                             kRsrcWord3);
}

// DMA one K or V tile (rows [tile*BC, tile*BC + BC) of a head) into the LDS tile at
// `dst`: the blocks slot, slot+NW, ... (< NB) of the wave whose place in the dealing
// order is `slot` (the wave index, or a rotation of it); src[i] is the lane's source
// offset for its i-th block (kDmaSkip: padding).  A device function (not a lambda)
// so that the host pass never sees the builtin.
//
// The LDS address of a block (M0 of the DMA) is the tile's offset plus the slot's
// block offset, formed here by a scalar add.  The slot's offset passes through an
// empty asm statement first: in an unrolled loop over several buffers the compiler
// would otherwise keep every (buffer, block) address live across the loop, run out
// of SGPRs and park them in VGPR lanes, so that each DMA costs a v_readlane (VALU
// issue time in the softmax phase) instead of an s_add.
template <int D, int NB, int PW, int NW, typename T>
__device__ __forceinline__ void stage_tile(const T* head, int tile, int nrows, char* dst,
                                           int slot, const int* src)
{
    const __amdgpu_buffer_rsrc_t r = rows_rsrc<D>(head, tile * 64, nrows);
    uint32_t slot_off = (uint32_t)__builtin_amdgcn_readfirstlane(slot * 1024);
    __asm__ volatile("" : "+s"(slot_off));
    const uint32_t tile_lds = (uint32_t)(uintptr_t)(lds_char*)dst;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int blk = slot + NW * i;
        if (blk < NB)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void*)(uintptr_t)(tile_lds + slot_off + NW * 1024 * i), 16, src[i], 0, 0, 0);
    }
}

// As stage_tile, with each DMA issued from inline assembly.  The compiler then does
// not see these writes into LDS, and so does not make the transposing LDS reads
// (ds_read_b64_tr_b16) that follow wait for every DMA the wave has in flight, which
// it does for DMA it can see.  The caller orders every read of a tile staged this way
// after a wait for its DMA (s_waitcnt vmcnt in every issuing wave, then a workgroup
// barrier), as the other waves' blocks require anyway.  M0 holds the LDS address of
// the block for the instruction that follows.
template <int D, int NB, int PW, int NW, typename T>
__device__ __forceinline__ void stage_tile_asm(const T* head, int tile, int nrows, char* dst,
                                               int wave, const int* src)
{
    // the resource of rows_rsrc as four words (base, stride 0, records, word 3), each
    // read from the first lane so that it sits in SGPRs however the code is optimised
    const int row0 = tile * 64;
    const int64_t n = nrows > row0 ? nrows - row0 : 0;
    const int64_t bytes = n * D * (int64_t)sizeof(T);
    const uint64_t base = (uint64_t)(uintptr_t)(head + (size_t)row0 * D);
    const u32x4 r = {(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xffffu)),
                     (uint32_t)__builtin_amdgcn_readfirstlane(bytes < kRsrcCap ? (int)bytes : kRsrcCap),
                     (uint32_t)kRsrcWord3};
#pragma unroll
    for (int i = 0; i < PW; ++i) {
        const int blk = wave + NW * i;
        if (blk < NB) {
            const int lds = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_char*)(dst + blk * 1024));
            __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                             :
                             : "s"(lds), "v"(src[i]), "s"(r)
                             : "memory");
        }
    }
}

// Transposing read of a 16-bit A operand (32 rows of the operand x 16 k-slots) from a
// row-major LDS tile whose rows are the k dimension: two ds_read_b64_tr_b16 at `p` and
// 8 rows further.  Lane (h = lane / 32, g = (lane / 16) % 2, j = lane % 16) passes
// p = tile + (4h + j / 4) * stride + 2 (16g + 4 (j % 4)) (+ 16 rows per 16-slot chunk,
// + 64 bytes per 32 columns); it receives column 16g + j (+ 32 per 64 bytes) with
// k-slots 8h + 4r + e holding rows 8r + 4h + e of the chunk (r = 0, 1; e = 0..3), the
// order in which a 32x32 accumulator rounded to T holds them.
template <int STR, typename V>
__device__ __forceinline__ V tr_operand(const char* p)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * STR));
    const s16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(V, w);
}

}  // namespace fa
