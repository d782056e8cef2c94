// dfc_gemm.hip - fused decode + matrix product Y = W X on gfx950, for W
// stored as a panel-layout DFC1 container (bf16 weights whose exponents are
// Huffman-coded, DFloat11 blog, sections 02 and 03).
//
// The weights are decoded as by the flat decoder's two phases, except that
// the first phase reads every chunk's code count from the container (the
// panel layout stores them) instead of decoding the chunk to count them: a
// wavefront scan of the counts gives each lane its write position, the
// write pass puts the exponents into LDS and checks that the lane's chunk
// held exactly its stored count.  The decoded values never reach HBM: each
// complete 32 x 16 sub-tile of W is assembled from its staged
// exponents and raw bytes straight into the A operand of one 32x32x16 bf16
// MFMA per 32 output columns, and the products accumulate in fp32 registers.
//
// Work decomposition: a workgroup takes whole panels (32 rows of W), a few
// wavefronts per panel, or, for matrices with too few panels to fill the
// GPU, a share of one panel's items; each wavefront decodes some items (32
// rows x panel_k columns) and accumulates their products in registers.
// A block of an item (64 chunks) decodes into the wavefront's staging area,
// whose start is the first sub-tile the block touches; the exponents of a
// sub-tile the block only begins are carried in registers into the next
// block's staging area.  The partial 32 x B products of a panel's wavefronts
// are then summed in LDS in wavefront order and written to Y with plain
// stores: no atomics, and the same bits on every run.  Only when a panel is
// shared by several workgroups are their sums added into Y (zeroed first)
// with fp32 atomics.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "dfc.h"
#include "dfc_decode_core.h"
#include "dfc_format.h"

namespace {

using bf16x8 = __attribute__((ext_vector_type(8))) __bf16;
using f32x16 = __attribute__((ext_vector_type(16))) float;

struct GemmArgs {
    const uint32_t *words;     // code stream (with its guard words)
    const uint32_t *offw;      // packed 5-bit chunk offsets
    const uint32_t *blockout;  // u32 out[n_blocks + 1], indices in panel order
    const uint32_t *items;     // (n_items + 1) x {first chunk, first block, code bits, 0}
    const uint8_t *counts;     // codes starting in every chunk (count_width(C) bytes each)
    const uint8_t *raw;        // raw bytes in panel order
    const uint8_t *lengths;    // the 256 code lengths (container bytes 256..511)
    const uint8_t *tables;     // tables from dfc_derive_tables, or null: derive them here
    const uint16_t *x;         // B vectors of K bf16: x[b K + k]
    void *xp;                  // X in operand order (pack_x_kernel), or null
    uint32_t xp_bytes;
    float *y;                  // B vectors of M fp32: y[b M + m]
    uint32_t words_bytes, offw_bytes, raw_bytes, x_bytes, y_bytes, counts_bytes;
    uint32_t n_panels, slices, panel_k, cols, rows, batch;
    uint32_t wpp, group;       // wavefronts per panel in a workgroup, panels per workgroup
    uint32_t split, rounds;    // workgroups per panel; rounds = ceil(n_panels / group) * split
    uint32_t tables_bytes, lut_bits, stage_bytes;
    uint32_t max_block;        // most codes a block may place (the staging capacity)
    uint32_t *status;
};

// Cache-policy operand of a buffer load on gfx950: the non-temporal bit.
constexpr int kLoadNT = 2;
// A byte offset from which every step of the prefetch (< 8 KB) stays past
// every range the launcher accepts (below kNowhere - 64 KB) and below 2^32.
constexpr uint32_t kFar = kNowhere - 8192u;

// Sub-tiles (512 values) whose raw bytes are prefetched into registers per
// block: a 64-chunk block of about 3 bits per code completes at most this
// many; the rest load when used.
template <int C>
struct GemmPrefetch {
    static constexpr int N = C >= 32 ? 10 : (C == 16 ? 7 : (C == 8 ? 4 : 3));
};

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8, v); }

// Position of an item (32 rows x panel_k columns of W, item q of the
// container): its first chunk and block, its block end, its code bits and
// its first element and column.
struct ItemPos {
    uint32_t q, c0, b0, b1, bits, e0, col0;
};

__device__ __forceinline__ ItemPos item_pos(const GemmArgs &g, uint32_t q) {
    const const_u32_ptr items = (const_u32_ptr)(g.items);
    ItemPos it;
    it.q = q;
    it.c0 = items[4 * q];
    it.b0 = items[4 * q + 1];
    it.bits = items[4 * q + 2];
    it.b1 = items[4 * q + 5];
    const uint32_t p = q / g.slices;
    it.col0 = (q % g.slices) * g.panel_k;
    it.e0 = 32u * (p * g.cols + it.col0);
    return it;
}

// The stored code count of chunk c: a byte up to C = 16, 16 bits at C = 32.
template <int C>
__device__ __forceinline__ uint32_t load_count(const __amdgpu_buffer_rsrc_t &cr, uint32_t c) {
    if constexpr (8 * C <= 255)
        return __builtin_amdgcn_raw_buffer_load_b8(cr, c, 0, 0);
    else
        return __builtin_amdgcn_raw_buffer_load_b16(cr, 2u * c, 0, 0);
}

// The B operand of column tile nt for the sub-tile at column k: lane L
// holds X[32 nt + L % 32][k + 8 (L / 32) .. + 8].  In place (x[b K + k],
// rows past B read as zeros), that is 32 pieces of 32 bytes, one per vector;
// from the packed copy (pack_x_kernel), one run of 1 KB.
template <int NT, bool XPACK>
__device__ __forceinline__ uint32_t x_offset(uint32_t xcol, uint32_t cols, uint32_t k, int nt, uint32_t lane) {
    if constexpr (XPACK)
        return (((k >> 4) * NT + uint32_t(nt)) * 64u + lane) * 16u;
    else
        return xcol + 2u * (32u * uint32_t(nt) * cols + k);
}

template <int NT, bool XPACK>
__device__ __forceinline__ u32x4 load_x(const __amdgpu_buffer_rsrc_t &xr, uint32_t xcol, uint32_t cols, uint32_t k,
                                        int nt, uint32_t lane) {
    return __builtin_amdgcn_raw_buffer_load_b128(xr, x_offset<NT, XPACK>(xcol, cols, k, nt, lane), 0, 0);
}

// X copied in the order load_x reads it: 16-byte unit ((k / 16) NT + nt)
// 64 + L holds X[32 nt + L % 32][k + 8 (L / 32) .. + 8] (zeros past B).
__global__ void pack_x_kernel(const uint16_t *x, uint32_t batch, uint32_t cols, uint32_t nt_count, uint4 *xp,
                              uint32_t units) {
    for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += gridDim.x * blockDim.x) {
        const uint32_t lane = u % 64u, nt = (u / 64u) % nt_count, kt = u / (64u * nt_count);
        const uint32_t n = 32u * nt + lane % 32u, k = 16u * kt + 8u * (lane / 32u);
        xp[u] = n < batch ? *reinterpret_cast<const uint4 *>(x + uint64_t(n) * cols + k) : make_uint4(0, 0, 0, 0);
    }
}

// The blocks of a wavefront's items (q0, q0 + qstep, ... below qend), one
// after another: each complete sub-tile is multiplied into acc.  The next
// block's stream words, chunk offsets, chunk counts and output range (in the
// same item or the next one) are requested before the current block is
// decoded, so their memory latency overlaps its decoding.  Returns false (and
// sets the status word) if a block's stored counts disagree with its block
// offsets or exceed the staging capacity (at once: acc then holds a partial
// sum), or if a chunk held a different number of codes than stored (noted
// per lane and reported after the last block, which keeps the write pass's
// result off the critical path of the loop).
template <int C, int NT, bool XPACK>
__device__ __forceinline__ bool gemm_items(const GemmArgs &g, uint32_t q0, uint32_t qstep, uint32_t qend,
                                           const Tables &t, uint8_t *stage, uint32_t lane,
                                           const __amdgpu_buffer_rsrc_t &words, const __amdgpu_buffer_rsrc_t &offw,
                                           const __amdgpu_buffer_rsrc_t &raw, const __amdgpu_buffer_rsrc_t &cr,
                                           const __amdgpu_buffer_rsrc_t &xr, uint32_t xcol, f32x16 (&acc)[NT]) {
    constexpr int PF = GemmPrefetch<C>::N;
    extern __shared__ __align__(16) uint8_t lds[];
    const const_u32_ptr blockout = (const_u32_ptr)(g.blockout);
    if (q0 >= qend) return true;
    ItemPos cur = item_pos(g, q0);
    uint32_t b = cur.b0;
    Chunk<C> ck;
    load_chunk<C>(words, offw, cur.c0 + lane, ck);
    uint32_t stored = load_count<C>(cr, cur.c0 + lane);
    uint32_t s_out = blockout[b], e_out = blockout[b + 1];
    wait_for(ck);
    wait_for(stored);
    u32x2 carry = {0u, 0u};
    bool miss = false;  // a chunk whose codes disagree with its stored count
    for (;;) {
        b = __builtin_amdgcn_readfirstlane(b);
        const uint32_t rs = s_out - cur.e0, base = rs & ~511u, lead = rs - base;
        const uint32_t total_want = e_out - s_out;
        // raw bytes only for the sub-tiles this block completes: the one it
        // only begins is carried as exponents, and the next block loads its
        // raw bytes
        const uint32_t rounds = (lead + total_want) >> 9;
        const uint32_t kcol = cur.col0 + 16u * (base >> 9);
        // (non-temporal: W's raw bytes are read once; X and the tables are
        // what the caches should keep); the loads past them go out of range
        // and return zeros, with no branch around them
        // (the step between sub-tiles goes into the loads' immediate offsets:
        // only the per-lane base is selected, between the sub-tiles' base
        // and kFar, from which every step stays out of range; the selection
        // is kept opaque so that the compiler does not fold the steps back
        // into it)
        static_assert(512 * (PF - 1) <= 8192, "prefetch steps from kFar");
        const uint32_t rbase = cur.e0 + base + 8u * lane;
        u32x2 R[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            uint32_t at = uint32_t(j) < rounds ? rbase : kFar;
            asm volatile("" : "+v"(at));
            R[j] = __builtin_amdgcn_raw_buffer_load_b64(raw, at + 512u * j, 0, kLoadNT);
        }
        // The X fragments of those sub-tiles too, so that their cache round
        // trips overlap the decoding instead of each product: all of them
        // with one column tile, those of the first XQ sub-tiles (every
        // column tile) with more, up to 16-byte chunks (the registers allow
        // no more).
        const uint32_t xbase = xcol + 2u * kcol;
        u32x4 XP[NT == 1 ? PF : 1];
#pragma unroll
        for (int j = 0; j < (NT == 1 ? PF : 0); ++j) {
            uint32_t at = uint32_t(j) < rounds ? xbase : kFar;
            asm volatile("" : "+v"(at));
            XP[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, at + 32u * j, 0, 0);
        }
        constexpr int XQ = NT > 1 && C <= 16 ? 2 : 0;
        u32x4 XQP[XQ > 0 ? XQ : 1][NT];
#pragma unroll
        for (int j = 0; j < XQ; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                XQP[j][nt] = __builtin_amdgcn_raw_buffer_load_b128(
                    xr, uint32_t(j) < rounds ? x_offset<NT, XPACK>(xcol, g.cols, kcol + 16u * j, nt, lane) : kFar, 0, 0);
        // the next block: this item's next, or the first of the next item
        const bool same = b + 1u < cur.b1;
        const bool more = same || cur.q + qstep < qend;
        ItemPos nit = cur;
        if (!same && more) nit = item_pos(g, cur.q + qstep);
        const uint32_t bn = same ? b + 1u : nit.b0;
        Chunk<C> nxt{};
        uint32_t s_nxt = 0, e_nxt = 0, stored_nxt = 0;
        if (more) {
            const uint32_t cn = nit.c0 + (bn - nit.b0) * kWave + lane;
            load_chunk<C>(words, offw, cn, nxt);
            stored_nxt = load_count<C>(cr, cn);
            s_nxt = blockout[bn];
            e_nxt = blockout[bn + 1];
        }
        // Zero the staging bytes this block ORs into, then put back the
        // exponents carried from the previous block in front of them.
        const uint32_t nz = min(lead + total_want + 8u, g.stage_bytes);
        for (uint32_t o = 16u * lane; o < nz; o += 16u * kWave)
            *reinterpret_cast<uint4 *>(stage + o) = make_uint4(0, 0, 0, 0);
        if (8u * lane < lead) *reinterpret_cast<u32x2 *>(stage + 8u * lane) = carry;

        const uint32_t ci = (b - cur.b0) * kWave + lane;  // item-relative chunk
        int start, end;
        chunk_span<C>(ck, cur.c0 + ci,
                      int(min(max(int64_t(cur.bits) - int64_t(ci) * (8 * C), int64_t(-1)), int64_t(8 * C + 32))),
                      start, end);
        // the write pass at a raised wave priority, the products at the normal
        // one (wavefronts that are decoding issue first)
        __builtin_amdgcn_s_setprio(1);
        const uint32_t cnt = start < end ? stored : 0u;
        const uint32_t incl = wave_inclusive_scan(cnt);
        const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
        const bool bad = (total != total_want) | (total_want > g.max_block) |
                   (__builtin_amdgcn_ballot_w64(cnt > 8u * C) != 0);
        uint32_t got = cnt;
        if (!bad && cnt) got = write_codes<C>(ck, start, end, lds_address(stage) + lead + (incl - cnt), t);
        miss |= (got != cnt) | ((start < end) & (cnt == 0));
        wait_for(R);
        if constexpr (NT == 1) wait_for(XP);
        wait_for(nxt);
        wait_for(stored_nxt);
        if (bad) {
            if (lane == 0 && g.status) atomicOr(g.status, kStatusCorrupt);
            return false;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        __builtin_amdgcn_s_setprio(0);
        // Complete sub-tiles: W operand from the staged exponents and the
        // raw bytes, X operand from global memory (cached); with several
        // column tiles, their X fragments are requested before their
        // products, so that their cache round trips overlap.
        const uint32_t extent = lead + total;
        // (equal to `rounds` here; kept opaque so that the compiler does not
        // hold the prefetch's conditions in registers across the write
        // pass to reuse them)
        uint32_t nfull = extent >> 9;
        asm volatile("" : "+s"(nfull));
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            if (uint32_t(j) < nfull) {
                const u32x2 E = *reinterpret_cast<const u32x2 *>(stage + 512u * j + 8u * lane);
                const bf16x8 A = as_bf16x8(assemble8(E, R[j]));
                u32x4 X[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if constexpr (NT == 1)
                        X[nt] = XP[j];
                    else if (j < XQ)
                        X[nt] = XQP[j < XQ ? j : 0][nt];
                    else
                        X[nt] = load_x<NT, XPACK>(xr, xcol, g.cols, kcol + 16u * j, nt, lane);
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, as_bf16x8(X[nt]), acc[nt], 0, 0, 0);
            }
        }
        for (uint32_t j = PF; j < nfull; ++j) {
            const u32x2 Rj = __builtin_amdgcn_raw_buffer_load_b64(raw, cur.e0 + base + 512u * j + 8u * lane, 0, kLoadNT);
            const u32x2 E = *reinterpret_cast<const u32x2 *>(stage + 512u * j + 8u * lane);
            const bf16x8 A = as_bf16x8(assemble8(E, Rj));
            u32x4 X[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                X[nt] = load_x<NT, XPACK>(xr, xcol, g.cols, kcol + 16u * j, nt, lane);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, as_bf16x8(X[nt]), acc[nt], 0, 0, 0);
        }
        // The sub-tile this block only began moves to the next block (an
        // item ends on a whole sub-tile, so nothing moves to the next item).
        const uint32_t tail = extent - 512u * nfull;
        carry = same && 8u * lane < tail ? *reinterpret_cast<const u32x2 *>(stage + 512u * nfull + 8u * lane)
                                         : u32x2{0u, 0u};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (!more) break;
        cur = nit;
        b = bn;
        ck = nxt;
        stored = stored_nxt;
        s_out = s_nxt;
        e_out = e_nxt;
    }
    if (__builtin_amdgcn_ballot_w64(miss) != 0) {
        if (lane == 0 && g.status) atomicOr(g.status, kStatusCorrupt);
        return false;
    }
    return true;
}

// Value r of lane L of a 32 x 32 accumulator tile goes to float4 slot
// 64 (r / 4) + L, element r % 4, of a wavefront's tile in LDS (see the
// reduction below for the rows and columns a slot holds).
__device__ __forceinline__ void put_tile(uint8_t *stage, uint32_t lane, const f32x16 &a) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4 *>(stage + 16u * (64u * r4 + lane)) =
            make_float4(a[4 * r4], a[4 * r4 + 1], a[4 * r4 + 2], a[4 * r4 + 3]);
}

// Workgroup of group x wpp wavefronts.  A round takes `group` consecutive
// panels (split == 1) or the part-th of split workgroups on one panel
// (group == 1); a panel's split * wpp wavefronts take its slices in turn:
// wavefront v of the panel takes slices v, v + split wpp, ...  Every staging
// area holds at least 4 KB, which the reduction reuses for one 32 x 32 fp32
// tile per wavefront.
template <int C, int NT, bool XPACK>
__global__ __launch_bounds__(512) void dfc_gemm_kernel(const GemmArgs g) {
    extern __shared__ __align__(16) uint8_t lds[];
    load_or_derive_tables(lds, g.tables, g.tables_bytes, g.lengths, g.lut_bits);
    const Tables t = tables_view(lds, g.lut_bits);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t wpp = g.wpp;
    const uint32_t pw = wave / wpp, sw = wave % wpp;  // panel in the round, first slice
    const uint32_t stage_off = g.tables_bytes + wave * g.stage_bytes;
    uint8_t *stage = lds + stage_off;
    const __amdgpu_buffer_rsrc_t words =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(g.words), 0, int(g.words_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t offw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(g.offw), 0, int(g.offw_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t raw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(g.raw), 0, int(g.raw_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t cr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(g.counts), 0, int(g.counts_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t xr =
        XPACK ? __builtin_amdgcn_make_buffer_rsrc(g.xp, 0, int(g.xp_bytes), kBufferConfig)
              : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(g.x), 0, int(g.x_bytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(g.y, 0, int(g.y_bytes), kBufferConfig);
    // B operand rows of this lane: column n = 32 nt + lane % 32 of X, k offset
    // 8 (lane / 32) inside the sub-tile (rows past B load zeros).
    const uint32_t xcol = 2u * (lane % 32u) * g.cols + 16u * (lane / 32u);

    const uint32_t stride = g.split * wpp;
    // the round count is the same for every wavefront of the workgroup
    for (uint32_t r = blockIdx.x; r < g.rounds; r += gridDim.x) {
        const uint32_t part = r % g.split;
        const uint32_t p = (r / g.split) * g.group + pw;
        f32x16 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
        if (p < g.n_panels)
            gemm_items<C, NT, XPACK>(g, p * g.slices + part * wpp + sw, stride, (p + 1) * g.slices, t, stage, lane,
                              words, offw, raw, cr, xr, xcol, acc);
        // D[i][j] of a 32x32 tile: i = 8 (r / 4) + 4 (lane / 32) + r % 4,
        // j = lane % 32.  Value r of lane L goes to slot 4 (64 (r / 4) + L) +
        // r % 4 of the wavefront's tile, so that element e of a float4 slot
        // holds rows 8 (e / 64) + 4 ((e % 64) / 32) + 0..3 of column e % 32.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt > 0) __syncthreads();  // the previous tile has been read
            put_tile(stage, lane, acc[nt]);
            __syncthreads();
            for (uint32_t e = sw * kWave + lane; e < 256u; e += wpp * kWave) {
                const uint8_t *slot = lds + g.tables_bytes + pw * wpp * g.stage_bytes + 16u * e;
                float4 v = *reinterpret_cast<const float4 *>(slot);
                for (uint32_t w = 1; w < wpp; ++w) {
                    const float4 u = *reinterpret_cast<const float4 *>(slot + w * g.stage_bytes);
                    v.x += u.x;
                    v.y += u.y;
                    v.z += u.z;
                    v.w += u.w;
                }
                const uint32_t n = 32u * uint32_t(nt) + e % 32u;
                const uint32_t m = 32u * p + 8u * (e / 64u) + 4u * ((e % 64u) / 32u);
                if (p < g.n_panels && n < g.batch) {
                    if (g.split == 1) {
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), yr, 4u * (n * g.rows + m), 0, 0);
                    } else {
                        float *yp = g.y + (uint64_t(n) * g.rows + m);
                        unsafeAtomicAdd(yp, v.x);
                        unsafeAtomicAdd(yp + 1, v.y);
                        unsafeAtomicAdd(yp + 2, v.z);
                        unsafeAtomicAdd(yp + 3, v.w);
                    }
                }
            }
        }
        __syncthreads();  // tiles read before the next round's staging
    }
}

__global__ void fill_zero_kernel(float *y, uint64_t n) {
    for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += uint64_t(gridDim.x) * blockDim.x)
        y[i] = 0.0f;
}

template <int C, int NT, bool XPACK>
dfc_status launch_gemm(const GemmArgs &proto, uint32_t max_block, hipStream_t stream) {
    GemmArgs g = proto;
    // staging: a carried partial sub-tile (< 512) + the block + spill, rounded
    // to 16, and at least one 32 x 32 fp32 tile for the reduction.  The spill
    // allows for one lane whose chunk holds more codes than stored (the
    // write pass stops at the chunk's end bit: at most 8C + 31 codes and
    // three past them, each ORed as two aligned dwords); the kernel then
    // reports it.
    const uint32_t stage = std::max(4096u, (511u + max_block + 8u * C + 48u + 15u) & ~15u);
    g.stage_bytes = stage;
    g.max_block = max_block;
    if (!allow_full_lds(reinterpret_cast<const void *>(&dfc_gemm_kernel<C, NT, XPACK>))) return DFC_EHIP;
    // about 8 wavefronts per workgroup: up to 8 per panel (one slice each
    // when the panel has 8 slices or fewer), several panels when it has few
    uint32_t wpp = std::min<uint32_t>(g.slices, 8u);
    uint32_t group = std::max<uint32_t>(1u, 8u / wpp);
    // the staging areas hold the table derivation's scratch before the first item
    const uint32_t scratch = g.tables ? 0u : derive_scratch_bytes(g.lut_bits);
    auto lds_for = [&](uint32_t w) { return size_t(g.tables_bytes) + std::max<size_t>(size_t(w) * stage, scratch); };
    while (wpp * group > 1 && lds_for(wpp * group) > kLdsBytes) {
        if (group > 1)
            --group;
        else
            --wpp;
    }
    const uint32_t waves = wpp * group;
    const size_t lds = lds_for(waves);
    if (lds > kLdsBytes) return DFC_EUNSUPPORTED;
    // Too few panels for the resident wavefronts: share each panel among
    // `split` workgroups, with as few slices per wavefront as the resident
    // count allows, spread evenly.
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&dfc_gemm_kernel<C, NT, XPACK>),
                                                     int(waves * kWave), lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const uint64_t resident = uint64_t(per_cu) * waves * uint64_t(device_cu_count());
    uint32_t split = 1;
    if (group == 1 && uint64_t(g.n_panels) * wpp < resident && g.slices > wpp) {
        const uint64_t want = std::min<uint64_t>(g.slices, dfc::ceil_div(resident, uint64_t(g.n_panels)));
        const uint64_t per_wave = dfc::ceil_div(uint64_t(g.slices), want);
        const uint64_t per_panel = dfc::ceil_div(uint64_t(g.slices), per_wave);
        split = uint32_t(dfc::ceil_div(per_panel, uint64_t(wpp)));
    }
    g.wpp = wpp;
    g.group = group;
    g.split = split;
    const uint64_t rounds = dfc::ceil_div(uint64_t(g.n_panels), uint64_t(group)) * split;
    if (rounds > 0x7fffffffull) return DFC_EUNSUPPORTED;
    g.rounds = uint32_t(rounds);
    // one workgroup per round: the hardware hands out the tail
    const uint32_t grid = g.rounds;
    if (split > 1)
        hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream, g.y, uint64_t(g.batch) * g.rows);
    if constexpr (XPACK) {
        const uint32_t units = g.xp_bytes / 16u;
        hipLaunchKernelGGL(pack_x_kernel, dim3(std::min<uint32_t>(1024u, (units + 255u) / 256u)), dim3(256), 0, stream,
                           g.x, g.batch, g.cols, uint32_t(NT), static_cast<uint4 *>(g.xp), units);
    }
    hipLaunchKernelGGL((dfc_gemm_kernel<C, NT, XPACK>), dim3(grid), dim3(waves * kWave), lds, stream, g);
    return hipGetLastError() == hipSuccess ? DFC_OK : DFC_EHIP;
}

template <int C>
dfc_status launch_gemm_c(const GemmArgs &g, uint32_t max_block, hipStream_t stream) {
    if (g.batch <= 32) return launch_gemm<C, 1, false>(g, max_block, stream);
    return g.xp ? launch_gemm<C, 2, true>(g, max_block, stream) : launch_gemm<C, 2, false>(g, max_block, stream);
}

}  // namespace

extern "C" {

uint64_t dfc_gemm_workspace_bytes(uint32_t batch, uint64_t cols) {
    return batch > 32 ? 2ull * 64ull * dfc::ceil_div(cols, 16) * 16ull : 0ull;
}

dfc_status dfc_decode_gemm(const void *w_blob_dev, const dfc_info *info, const void *tables_dev, const uint16_t *x_dev,
                           uint32_t batch, float *y_dev, void *workspace_dev, uint64_t workspace_bytes,
                           uint32_t *status_dev, void *stream) {
    if (!info || !w_blob_dev || !x_dev || !y_dev) return DFC_EINVAL;
    if (batch < 1 || batch > DFC_GEMM_MAX_BATCH) return DFC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(w_blob_dev) & 255u) || (reinterpret_cast<uintptr_t>(x_dev) & 15u) ||
        (reinterpret_cast<uintptr_t>(y_dev) & 3u) || (reinterpret_cast<uintptr_t>(tables_dev) & 15u) ||
        (reinterpret_cast<uintptr_t>(workspace_dev) & 15u))
        return DFC_EINVAL;
    const dfc_info &in = *info;
    if (in.layout != DFC_LAYOUT_PANEL || in.panel_rows != dfc::kPanelRows || in.lanes_per_block != 64)
        return DFC_EUNSUPPORTED;
    const uint32_t C = in.chunk_bytes;
    if (C != 4 && C != 8 && C != 16 && C != 32) return DFC_EINVAL;
    if (in.lut_bits < 8 || in.lut_bits > 12 || in.min_len < 1) return DFC_EINVAL;
    if (in.max_block_elems > 64u * dfc::ceil_div(8ull * C, in.min_len)) return DFC_EINVAL;
    const uint64_t limit = kNowhere - 64u * 1024u;
    if (in.counts_bytes < dfc::count_width(C) * in.n_chunks) return DFC_EINVAL;
    if (in.words_bytes > limit || in.offsets_bytes > limit || in.raw_bytes > limit || in.counts_bytes > limit ||
        2ull * DFC_GEMM_MAX_BATCH * in.cols > limit || 4ull * DFC_GEMM_MAX_BATCH * in.rows > limit)
        return DFC_EUNSUPPORTED;
    const uint8_t *base = static_cast<const uint8_t *>(w_blob_dev);
    GemmArgs g;
    std::memset(&g, 0, sizeof(g));
    g.words = reinterpret_cast<const uint32_t *>(base + in.off_words);
    g.offw = reinterpret_cast<const uint32_t *>(base + in.off_offsets);
    g.blockout = reinterpret_cast<const uint32_t *>(base + in.off_blockout);
    g.items = reinterpret_cast<const uint32_t *>(base + in.off_panels);
    g.counts = base + in.off_counts;
    g.counts_bytes = uint32_t(in.counts_bytes);
    g.raw = base + in.off_raw;
    g.lengths = base + dfc::hdr::lengths;
    g.tables = static_cast<const uint8_t *>(tables_dev);
    g.x = x_dev;
    g.y = y_dev;
    g.words_bytes = uint32_t(in.words_bytes);
    g.offw_bytes = uint32_t(in.offsets_bytes);
    g.raw_bytes = uint32_t(in.raw_bytes);
    g.x_bytes = uint32_t(2ull * batch * in.cols);
    g.y_bytes = uint32_t(4ull * batch * in.rows);
    g.n_panels = uint32_t(in.rows / dfc::kPanelRows);
    g.panel_k = in.panel_k;
    g.slices = uint32_t(dfc::ceil_div(in.cols, in.panel_k));
    g.cols = uint32_t(in.cols);
    g.rows = uint32_t(in.rows);
    g.batch = batch;
    g.tables_bytes = uint32_t(dfc::tables_bytes(in.lut_bits));
    const uint64_t ws = dfc_gemm_workspace_bytes(batch, in.cols);
    if (workspace_dev && ws) {
        if (workspace_bytes < ws) return DFC_ESIZE;
        g.xp = workspace_dev;
        g.xp_bytes = uint32_t(ws);
    }
    g.lut_bits = in.lut_bits;
    g.status = status_dev;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (C) {
        case 4: return launch_gemm_c<4>(g, in.max_block_elems, st);
        case 8: return launch_gemm_c<8>(g, in.max_block_elems, st);
        case 16: return launch_gemm_c<16>(g, in.max_block_elems, st);
        default: return launch_gemm_c<32>(g, in.max_block_elems, st);
    }
}

}  // extern "C"
