// dfc_decode.hip - gfx950 decoder for DFC1 containers and its C-ABI launchers.
//
// DFloat11 blog ("70% Size, 100% Accuracy ... (DFloat11)"), section 03:
//   item 1: compact hierarchical lookup tables in on-chip memory find code
//           boundaries fast -> the first-level k-bit tables (step, symbols,
//           boundary mask) and the per-length canonical tables for longer
//           codes live in LDS: every workgroup derives them from the 256
//           code lengths, or copies the image dfc_derive_tables prepared
//           once per container;
//   item 2: a two-phase kernel; in phase one threads agree on read and write
//           positions through small auxiliary variables, phase two rebuilds
//           the weights -> per-chunk start offsets and per-block output
//           offsets come from the container, each lane counts the codes of
//           its chunk, a wavefront prefix scan turns counts into write
//           positions, the exponents go to LDS and are merged with the raw
//           bytes into bf16 with coalesced 16-byte stores.  Containers in the
//           padded layout have no chunk offsets: there every chunk starts
//           with a code and ends with its last whole code.
//
// Work decomposition: one lane per chunk (C bytes of code stream), one
// wavefront (64 lanes) per block of 64 chunks.  Workgroups are persistent:
// the grid is sized to the resident capacity of the GPU and each matrix gets
// a share of it.  A matrix's blocks are cut into runs of a few consecutive
// blocks, dealt out to its V wavefronts in turn (wavefront v takes runs v,
// v + V, v + 2V, ...), so that the wavefronts resident at one time read and
// write neighbouring parts of the streams: memory serves that faster than as
// many streams far apart.  A wavefront decodes block after block, within a
// run and across runs, while the next block's stream words, offsets and
// output range are in flight.  All decoding is integer work on bit patterns.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <vector>

#include "dfc.h"
#include "dfc_ans_launch.h"
#include "dfc_decode_core.h"
#include "dfc_format.h"

namespace {

struct ItemArgs {
    const uint32_t *words;     // code stream (with its guard words)
    const uint32_t *offw;      // packed 5-bit chunk offsets
    const uint32_t *blockout;  // u32 out[n_blocks + 1]
    const uint8_t *raw;        // raw bytes (sign << 7 | mantissa), padded to 16
    const uint8_t *lengths;    // the 256 code lengths (container bytes 256..511)
    const uint8_t *tables;     // tables from dfc_derive_tables, or null: derive them here
    uint16_t *dst;             // bf16 output
    uint64_t total_bits;
    uint32_t words_bytes, offw_bytes, raw_bytes, dst_bytes;  // buffer ranges
    uint32_t n_blocks;
    uint32_t wg_begin;         // first workgroup of this item in the grid
    uint32_t wgs;              // workgroups of this item
    uint32_t tables_bytes;     // LDS image of the derived tables, a multiple of 16
    uint32_t lut_bits;
    uint32_t run;              // blocks per run (see the kernel)
};

struct Buffers {
    __amdgpu_buffer_rsrc_t words, offw, raw, dst;
};

__device__ __forceinline__ Buffers make_buffers(const ItemArgs &a) {
    Buffers r;
    r.words = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(a.words), 0, int(a.words_bytes), kBufferConfig);
    r.offw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(a.offw), 0, int(a.offw_bytes), kBufferConfig);
    r.raw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.raw), 0, int(a.raw_bytes), kBufferConfig);
    r.dst = __builtin_amdgcn_make_buffer_rsrc(a.dst, 0, int(a.dst_bytes), kBufferConfig);
    return r;
}

struct BatchArgs {
    ItemArgs item[DFC_MAX_BATCH];
    uint32_t count;
    uint32_t stage_bytes;  // LDS exponent staging per wavefront (multiple of 16)
    uint32_t *status;
};

// Rounds of raw-byte octets (512 values per wavefront per round) prefetched
// into registers before decoding: enough for a block of 64 chunks at about
// 4 bits per code.
template <int C>
struct Prefetch {
    static constexpr int N = C >= 32 ? 12 : C / 2;
};

// Wavefronts per SIMD the register budget is sized for (512 VGPRs per lane
// shared by the resident wavefronts).  With deferred stores (below) the
// assembled rounds held in registers allow at most 128 VGPRs and 4
// wavefronts (C = 16 uses all of them; C = 4 and 8 fit 7 and 5); without
// them 64 VGPRs give 8 (the 32-byte chunk path needs more and settles for
// 5).  The launcher picks the build per chunk size and job (launch_group).
template <int C, bool Defer>
struct Occupancy {
    static constexpr int kWavesPerSimd = Defer ? 4 : (C >= 32 ? 5 : 8);
};

// Output rounds.  A wavefront decodes its runs of consecutive blocks one
// after another and writes each run's output in rounds of 512 values (1 KB
// of bf16, one 16-byte store per lane) aligned to multiples of 512 in the
// output: a block's exponents are
// staged in LDS behind the values still pending from the blocks before it
// (fewer than 512, kept in registers in between), every complete round is
// merged with its raw bytes and stored (the first few during the next
// block's write pass), and the rest is carried on.  Only
// the first and last round of a run can be partial; values outside the
// run's [lo, hi) are not written (an octet cut by lo or hi goes out with
// 16-bit stores).
constexpr uint32_t kRound = 512;

// One round of 512 values from output index base (a multiple of 512): this
// lane's octet v0 = base + 8 lane, exponents E, raw bytes R.  `edge` is
// uniform: false when the whole round lies inside [lo, hi).
__device__ __forceinline__ void store_round(const Buffers &bf, uint32_t base, uint32_t lane, const u32x2 &E,
                                            const u32x2 &R, bool edge, uint32_t lo, uint32_t hi) {
    const u32x4 o = assemble8(E, R);
    const uint32_t v0 = base + 8u * lane;
    if (!edge) {
        __builtin_amdgcn_raw_buffer_store_b128(o, bf.dst, 2u * v0, 0, 0);
        return;
    }
    const bool full = v0 >= lo && v0 + 8u <= hi;
    __builtin_amdgcn_raw_buffer_store_b128(o, bf.dst, full ? 2u * v0 : kNowhere, 0, 0);
    if (!full && v0 + 8u > lo && v0 < hi) {
        const uint32_t v[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t at = (v0 + q >= lo && v0 + q < hi ? 2u * v0 : kNowhere) + 2u * uint32_t(q);
            __builtin_amdgcn_raw_buffer_store_b16(uint16_t(v[q >> 1] >> (16 * (q & 1))), bf.dst, at, 0, 0);
        }
    }
}

// Raw bytes of this lane's octet of the round at base, or nothing (zeros, no
// memory access) for an octet wholly outside [lo, hi).
__device__ __forceinline__ u32x2 load_raw_octet(const Buffers &bf, uint32_t base, uint32_t lane, uint32_t lo,
                                                uint32_t hi) {
    const uint32_t v0 = base + 8u * lane;
    return __builtin_amdgcn_raw_buffer_load_b64(bf.raw, v0 + 8u > lo && v0 < hi ? v0 : kNowhere, 0, 0);
}

// The values still pending in the carry registers, [base, hi) minus what
// lies below lo, stored as a last (partial) round.
__device__ __forceinline__ void flush_round(const Buffers &bf, uint32_t base, uint32_t lane, const u32x2 &carry,
                                            uint32_t lo, uint32_t hi) {
    if (hi <= base) return;
    const u32x2 R = load_raw_octet(bf, base, lane, lo, hi);
    store_round(bf, base, lane, carry, R, true, lo, hi);
}

template <int C, bool Padded, bool Defer>
__global__ __launch_bounds__(1024, (Occupancy<C, Defer>::kWavesPerSimd)) void dfc_decode_kernel(const BatchArgs args) {
    extern __shared__ __align__(16) uint8_t lds[];
    constexpr int PF = Prefetch<C>::N;
    const uint32_t wg = blockIdx.x;
    uint32_t it = 0;
    for (uint32_t k = 1; k < args.count; ++k)
        if (wg >= args.item[k].wg_begin) it = k;
    const ItemArgs a = args.item[it];
    const Buffers bf = make_buffers(a);
    const const_u32_ptr blockout = (const_u32_ptr)(a.blockout);

    const uint32_t waves = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane = threadIdx.x % kWave;
    const uint32_t stage_off = a.tables_bytes + wave * args.stage_bytes;
    uint8_t *stage = lds + stage_off;
    const uint32_t stage_addr = lds_address(stage);  // its LDS address
    // this wavefront's first run, [b, b_end), and the matrix's run count;
    // runs go to the first wavefront of every workgroup, then to the
    // second, ..., so that every workgroup gets an even share
    const uint32_t run = a.run;
    const uint32_t V = a.wgs * waves;
    const uint32_t nruns = (a.n_blocks + run - 1u) / run;
    uint32_t r = wave * a.wgs + (wg - a.wg_begin);
    uint32_t b = min(r, nruns) * run;
    uint32_t b_end = min(b + run, a.n_blocks);

    // The first block's stream words and output range are requested before
    // the tables are derived (the derivation's barriers wait for LDS only),
    // so their memory latency overlaps it.
    Chunk<C> cur{};
    uint32_t s_out = 0, e_out = 0;
    if (b < b_end) {
        load_chunk<C, !Padded>(bf.words, bf.offw, b * kWave + lane, cur);
        s_out = blockout[b];
        e_out = blockout[b + 1];
    }
    load_or_derive_tables(lds, a.tables, a.tables_bytes, a.lengths, a.lut_bits);
    const Tables t = tables_view(lds, a.lut_bits);
    if (b >= b_end) return;
    // Resident on entry, as it is on every later iteration (see wait_for).
    wait_for(cur);

    // run state: rounds start at base (a multiple of 512); values below lo
    // belong to another run; the carry holds [base, s_out).  Every run
    // starts this way.
    uint32_t base = s_out & ~(kRound - 1u), lo = s_out;
    u32x2 carry = {0u, 0u};
    // Deferred stores: the first DEF complete rounds of a block are assembled
    // into registers and stored during the next block's write pass, one per
    // stream word, so that the wavefront's stores are spread over its decode
    // instead of leaving in one burst (O[j] is round pbase + 512 j; npend
    // of them are pending, the first only if it was not an edge round).
    // Without Defer, DEF is 0 and every round is stored when assembled.
    constexpr int DEF = !Defer ? 0 : C >= 32 ? 2 : (C / 4 + 1 < Prefetch<C>::N ? C / 4 + 1 : Prefetch<C>::N);
    u32x4 O[DEF > 0 ? DEF : 1];
    uint32_t pbase = 0, npend = 0;
    bool pfirst_edge = false;
    for (;;) {
        // the block index is the same in every lane
        b = __builtin_amdgcn_readfirstlane(b);
        const uint32_t lead = s_out - base;  // pending values, < 512
        const uint32_t want = e_out - s_out;
        const uint32_t rounds = (lead + want) / kRound;  // rounds this block completes
        // the next block: this run's next, or the first of the wavefront's next run
        const bool in_run = b + 1u < b_end;
        const uint32_t rn = in_run ? r : r + V;
        const uint32_t bn = in_run ? b + 1u : min(rn, nruns) * run;
        const bool more = in_run || rn < nruns;
        // raw bytes of those rounds (the first PF of them) per lane, and at
        // the end of a run those of its last, partial round; the loads of
        // rounds past them are branched around (a load whose lanes all lie
        // out of range would still take a slot in the address queue)
        const uint32_t rounds_raw = rounds + (in_run ? 0u : 1u);
        u32x2 R[PF];
        const uint32_t nraw = __builtin_amdgcn_readfirstlane(rounds_raw);
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            R[j] = u32x2{0u, 0u};
            if (uint32_t(j) < nraw) R[j] = load_raw_octet(bf, base + kRound * j, lane, lo, e_out);
        }
        // next block's stream words, offsets and output range
        Chunk<C> nxt{};
        uint32_t s_nxt = 0, e_nxt = 0;
        if (more) {
            load_chunk<C, !Padded>(bf.words, bf.offw, bn * kWave + lane, nxt);
            s_nxt = blockout[bn];
            e_nxt = blockout[bn + 1];
        }
        // Zero the staging bytes this block ORs its exponents into (the
        // pending values, the block's, and the spill of its last lookup),
        // then put the pending values back in front.
        const uint32_t nz = min(lead + want + 8u, args.stage_bytes);
        for (uint32_t o = 16u * lane; o < nz; o += 16u * kWave)
            *reinterpret_cast<uint4 *>(stage + o) = make_uint4(0, 0, 0, 0);
        if (8u * lane < lead) *reinterpret_cast<u32x2 *>(stage + 8u * lane) = carry;

        const uint32_t chunk = b * kWave + lane;
        // Stream bits from this lane's chunk to the end of the stream: only
        // the last block needs them per lane (a uniform 64-bit test, then 32 bits).
        const int64_t block_left = int64_t(a.total_bits) - int64_t(uint64_t(b) * (uint64_t(kWave) * 8u * C));
        const int bits_left = block_left >= int64_t(kWave) * (8 * C + 32)
                                  ? (8 * C + 32)
                                  : max(int(block_left) - int(lane) * (8 * C), -1);
        int start = 0, end;
        if constexpr (Padded)
            end = min(8 * C, bits_left);
        else
            chunk_span<C>(cur, chunk, bits_left, start, end);

        // The count and write passes run at a raised wave priority, so that
        // the wavefronts that are decoding get issue slots ahead of those
        // that are storing; the store rounds drop back to the normal priority.
        __builtin_amdgcn_s_setprio(1);
        uint32_t cnt = 0;
        if (start < end) cnt = Padded ? count_codes_padded<C>(cur, end, t) : count_codes<C>(cur, start, end, t);
        const uint32_t incl = wave_inclusive_scan(cnt);
        const uint32_t total = __builtin_amdgcn_readlane(incl, kWave - 1);
        // A chunk of 8C bits holds at most 8C code starts; anything else (or
        // a total that disagrees with the block offsets) means a corrupt stream.
        const bool bad = (total != want) | (__builtin_amdgcn_ballot_w64(cnt > 8u * C) != 0);
        // The previous block's deferred rounds go out during this block's
        // write pass, after its loads have arrived (a store issued before
        // them would make their wait include the store).  Every lane runs
        // the write pass (a lane without codes does no lookup), since every
        // lane stores its octet of each round.
        auto hook = [&](int w) {
            if (uint32_t(w) < npend && (w > 0 || !pfirst_edge))
                __builtin_amdgcn_raw_buffer_store_b128(O[w < DEF ? w : 0], bf.dst,
                                                       2u * (pbase + kRound * uint32_t(w) + 8u * lane), 0, 0);
        };
        if constexpr (Defer) {
            // Everything prefetched must be in registers before the first
            // store, on every path to the next block.
            wait_for(R);
            wait_for(nxt);
            if (!bad) {
                if constexpr (Padded)
                    write_codes_padded<C>(cur, end, cnt, stage_addr + lead + (incl - cnt), t, hook);
                else
                    write_codes<C>(cur, start, end, stage_addr + lead + (incl - cnt), t, hook);
            } else {
                for (int w = 0; w <= C / 4; ++w) hook(w);
            }
        } else {
            // no stores in the write pass: the loads stay in flight during it
            if (!bad && cnt) {
                if constexpr (Padded)
                    write_codes_padded<C>(cur, end, cnt, stage_addr + lead + (incl - cnt), t);
                else
                    write_codes<C>(cur, start, end, stage_addr + lead + (incl - cnt), t);
            }
            wait_for(R);
            wait_for(nxt);
        }
        npend = 0;
        __builtin_amdgcn_s_setprio(0);
        if (bad) {
            // the block stays unwritten: store what is pending before it and
            // start a new run after it
            if (lane == 0 && args.status) atomicOr(args.status, kStatusCorrupt);
            flush_round(bf, base, lane, carry, lo, s_out);
            base = e_out & ~(kRound - 1u);
            lo = e_out;
            carry = u32x2{0u, 0u};
        } else {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // complete rounds, kept for the next block's write pass to store
            // (the first round of a run, which can start below lo, goes out now)
            pfirst_edge = base < lo;
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                if (uint32_t(j) < rounds) {
                    const u32x2 E = *reinterpret_cast<const u32x2 *>(stage + kRound * j + 8u * lane);
                    if (j == 0 && pfirst_edge)
                        store_round(bf, base, lane, E, R[0], true, lo, e_out);
                    else if (j < DEF)
                        O[j < DEF ? j : 0] = assemble8(E, R[j]);
                    else
                        store_round(bf, base + kRound * j, lane, E, R[j], false, lo, e_out);
                }
            }
            pbase = base;
            npend = min(rounds, uint32_t(DEF));
            for (uint32_t j = PF; j < rounds; ++j) {
                const u32x2 Rj = load_raw_octet(bf, base + kRound * j, lane, lo, e_out);
                const u32x2 E = *reinterpret_cast<const u32x2 *>(stage + kRound * j + 8u * lane);
                store_round(bf, base + kRound * j, lane, E, Rj, base + kRound * j < lo, lo, e_out);
            }
            // the values of the round this block only began move on
            const uint32_t tail = lead + want - kRound * rounds;
            carry = 8u * lane < tail ? *reinterpret_cast<const u32x2 *>(stage + kRound * rounds + 8u * lane)
                                     : u32x2{0u, 0u};
            base += kRound * rounds;
            if (!in_run && base < e_out) {
                // the run ends inside this round: it goes out now, with the
                // raw bytes loaded at the block's start
                u32x2 Rt = {0u, 0u};
#pragma unroll
                for (int j = 0; j < PF; ++j)
                    if (uint32_t(j) == rounds) Rt = R[j];
                if (rounds >= uint32_t(PF)) Rt = load_raw_octet(bf, base, lane, lo, e_out);
                store_round(bf, base, lane, carry, Rt, true, lo, e_out);
            }
        }
        // The next block reuses this wavefront's staging area.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (!more) {
#pragma unroll
            for (int w = 0; w < DEF; ++w) hook(w);
            break;
        }
        if (!in_run) {
            // a new run: nothing pending in front of its first block (the
            // deferred rounds of this block are complete and go out during
            // the next block's write pass as usual)
            r = rn;
            b_end = min(bn + run, a.n_blocks);
            base = s_nxt & ~(kRound - 1u);
            lo = s_nxt;
            carry = u32x2{0u, 0u};
        }
        cur = nxt;
        b = bn;
        s_out = s_nxt;
        e_out = e_nxt;
    }
}

// The decode tables as one workgroup derives them, copied out of LDS (for
// inspection; the decoders keep them in LDS).
__global__ __launch_bounds__(1024) void derive_tables_kernel(const uint8_t *lengths, uint32_t lut_bits,
                                                             uint32_t tables_bytes, uint8_t *dst) {
    extern __shared__ __align__(16) uint8_t lds[];
    derive_tables(lds, lds + tables_bytes, lengths, lut_bits);
    for (uint32_t o = 16u * threadIdx.x; o < tables_bytes; o += 16u * blockDim.x)
        *reinterpret_cast<uint4 *>(dst + o) = *reinterpret_cast<const uint4 *>(lds + o);
}

// ------------------------------------------------------------------ launch

// Set by dfc_set_launch, read by every launch (possibly on other threads).
struct LaunchCfg {
    std::atomic<uint32_t> waves{0}, blocks_per_wave{0}, stores{0}, run{0};
} g_launch;

// Blocks per run when none is set: about 6,144 output values (two blocks
// of Gaussian-like weights at C = 16, eight at C = 4), at least 2 and at
// most 16 blocks, and no more than a quarter of the blocks each wavefront
// gets, so that the last round of runs leaves the wavefronts evenly loaded
// (a small matrix, under 4 blocks per wavefront, goes one block per run and
// keeps every wavefront busy).  Short runs at small C spend too much of
// each run on its two partial rounds: runs of 8 instead of 2 decode the
// stress tensors at C = 4 5-6% faster.
uint32_t auto_run(uint64_t blocks, uint64_t wavefronts, uint64_t n) {
    const uint64_t per_block = std::max<uint64_t>(1, n / std::max<uint64_t>(1, blocks));
    const uint64_t run = std::min<uint64_t>(16, std::max<uint64_t>(2, (6144 + per_block / 2) / per_block));
    return uint32_t(std::min<uint64_t>(run, std::max<uint64_t>(1, blocks / (4 * wavefronts))));
}

// Split `slots` workgroups across items so that the largest per-workgroup
// block count is as small as possible (each item gets at least one).
std::vector<uint32_t> share_workgroups(const std::vector<uint64_t> &blocks, uint64_t slots, uint32_t per_wg_min) {
    const size_t m = blocks.size();
    std::vector<uint32_t> g(m, 1);
    uint64_t used = m;
    auto load = [&](size_t i) { return dfc::ceil_div(blocks[i], g[i]); };
    while (used < slots) {
        size_t best = 0;
        for (size_t i = 1; i < m; ++i)
            if (load(i) > load(best)) best = i;
        if (load(best) <= per_wg_min) break;
        g[best]++;
        used++;
    }
    return g;
}

// The launch geometry of one build of the decoder for a group of items: the
// workgroup shape and LDS, each item's workgroups, and the most blocks any
// wavefront decodes in sequence (the launch's critical path).
struct Plan {
    uint32_t waves = 0, lds = 0, stage = 0;
    std::vector<uint32_t> live, g, run;
    uint64_t crit = 0;
};

template <int C, bool Padded, bool Defer>
dfc_status plan_group(const dfc_batch_item *items, const uint32_t *idx, uint32_t count, Plan &pl) {
    uint32_t max_tables = 0, max_block = 0, max_scratch = 0;
    std::vector<uint64_t> blocks;
    for (uint32_t k = 0; k < count; ++k) {
        const dfc_info &in = *items[idx[k]].info;
        if (in.n_blocks == 0) continue;
        pl.live.push_back(idx[k]);
        blocks.push_back(in.n_blocks);
        max_tables = std::max<uint32_t>(max_tables, uint32_t(dfc::tables_bytes(in.lut_bits)));
        if (!items[idx[k]].tables_dev) max_scratch = std::max<uint32_t>(max_scratch, derive_scratch_bytes(in.lut_bits));
        max_block = std::max(max_block, in.max_block_elems);
    }
    if (pl.live.empty()) return DFC_OK;
    const void *kernel = reinterpret_cast<const void *>(&dfc_decode_kernel<C, Padded, Defer>);
    // staging: pending values of the round in progress (< 512) + the block's
    // values + the spill of its last lookup, rounded to 16
    const uint32_t stage = (511u + max_block + 32u + 15u) & ~15u;
    if (!allow_full_lds(kernel)) return DFC_EHIP;
    // LDS of a workgroup of w wavefronts: the tables, then the staging
    // areas, which hold the derivation's scratch before the first block.
    auto lds_for = [&](uint32_t w) { return max_tables + std::max(w * stage, max_scratch); };
    // Resident workgroups per CU for w wavefronts each, under both the LDS
    // and the register budget.
    // The answer for the last LDS size asked is kept per workgroup shape
    // ((LDS << 32) | (count + 1), 0 = none), since every launch asks again.
    static std::atomic<uint64_t> memo[kMaxWaves + 1];
    auto resident = [&](uint32_t w) -> int {
        const uint32_t lds = lds_for(w);
        if (lds > kLdsBytes) return 0;
        const uint64_t m = memo[w].load(std::memory_order_relaxed);
        if (m && uint32_t(m >> 32) == lds) return int(uint32_t(m)) - 1;
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, int(w * kWave), size_t(lds)) != hipSuccess)
            per_cu = int(kLdsBytes / lds);
        memo[w].store((uint64_t(lds) << 32) | uint32_t(per_cu + 1), std::memory_order_relaxed);
        return per_cu;
    };
    // waves per workgroup: the most resident wavefronts per CU, then the
    // smaller workgroup (the dispatcher spreads more, smaller workgroups
    // more evenly; the whole model decodes about 1% faster with two
    // workgroups of 8 wavefronts per CU than with one of 16)
    uint32_t waves = g_launch.waves.load(std::memory_order_relaxed);
    const uint32_t blocks_per_wave = g_launch.blocks_per_wave.load(std::memory_order_relaxed);
    if (!waves) {
        uint32_t best = 0;
        for (uint32_t w = 4; w <= kMaxWaves; ++w) {
            const uint32_t r = uint32_t(std::max(0, resident(w))) * w;
            if (r > best) {
                best = r;
                waves = w;
            }
        }
    }
    if (!waves) waves = 1;
    while (waves > 1 && lds_for(waves) > kLdsBytes) --waves;
    if (lds_for(waves) > kLdsBytes) return DFC_EUNSUPPORTED;
    int per_cu = resident(waves);
    if (per_cu <= 0) per_cu = 1;
    uint64_t slots = uint64_t(per_cu) * uint64_t(device_cu_count());
    if (blocks_per_wave) {
        // fixed work per workgroup instead of filling the machine exactly
        uint64_t total = 0;
        for (uint64_t nb : blocks) total += dfc::ceil_div(nb, uint64_t(waves) * blocks_per_wave);
        slots = total;
    }
    pl.g = share_workgroups(blocks, std::max<uint64_t>(slots, pl.live.size()), waves);
    pl.waves = waves;
    pl.lds = lds_for(waves);
    pl.stage = stage;
    // Workgroups beyond what the machine holds at once run after others
    // finish: count them as further blocks in sequence.
    uint64_t wgs = 0;
    const uint32_t run_set = g_launch.run.load(std::memory_order_relaxed);
    for (size_t k = 0; k < blocks.size(); ++k) {
        const uint64_t per_wg = dfc::ceil_div(blocks[k], uint64_t(pl.g[k]));
        const uint64_t wgs_k = dfc::ceil_div(blocks[k], per_wg);
        const uint64_t wavefronts = wgs_k * waves;
        const uint32_t run = run_set ? run_set : auto_run(blocks[k], wavefronts, items[pl.live[k]].info->n);
        pl.run.push_back(run);
        pl.crit = std::max(pl.crit, dfc::ceil_div(dfc::ceil_div(blocks[k], uint64_t(run)), wavefronts) * run);
        wgs += wgs_k;
    }
    pl.crit *= dfc::ceil_div(wgs, uint64_t(per_cu) * uint64_t(device_cu_count()));
    return DFC_OK;
}

template <int C, bool Padded, bool Defer>
dfc_status launch_planned(const dfc_batch_item *items, const Plan &pl, uint32_t *status, hipStream_t stream) {
    if (pl.live.empty()) return DFC_OK;
    BatchArgs args;
    std::memset(&args, 0, sizeof(args));
    uint32_t wg = 0;
    for (size_t k = 0; k < pl.live.size(); ++k) {
        const dfc_batch_item &bi = items[pl.live[k]];
        const dfc_info &in = *bi.info;
        const uint8_t *base = static_cast<const uint8_t *>(bi.blob_dev);
        ItemArgs &a = args.item[k];
        a.words = reinterpret_cast<const uint32_t *>(base + in.off_words);
        a.offw = reinterpret_cast<const uint32_t *>(base + in.off_offsets);
        a.blockout = reinterpret_cast<const uint32_t *>(base + in.off_blockout);
        a.raw = base + in.off_raw;
        a.lengths = base + dfc::hdr::lengths;
        a.tables = static_cast<const uint8_t *>(bi.tables_dev);
        a.dst = bi.dst_dev;
        a.words_bytes = uint32_t(in.words_bytes);
        a.offw_bytes = uint32_t(in.offsets_bytes);
        a.raw_bytes = uint32_t(in.raw_bytes);
        a.dst_bytes = uint32_t(2 * in.n);
        a.total_bits = in.total_bits;
        a.n_blocks = uint32_t(in.n_blocks);
        const uint64_t per_wg = dfc::ceil_div(in.n_blocks, pl.g[k]);
        a.wgs = uint32_t(dfc::ceil_div(in.n_blocks, per_wg));
        a.wg_begin = wg;
        a.tables_bytes = uint32_t(dfc::tables_bytes(in.lut_bits));
        a.lut_bits = in.lut_bits;
        a.run = pl.run[k];
        wg += a.wgs;
    }
    args.count = uint32_t(pl.live.size());
    args.stage_bytes = pl.stage;
    args.status = status;
    dfc_decode_kernel<C, Padded, Defer><<<dim3(wg), dim3(pl.waves * kWave), pl.lds, stream>>>(args);
    return hipGetLastError() == hipSuccess ? DFC_OK : DFC_EHIP;
}

// One launch for a group of items of one chunk size and layout.  The
// deferred build's registers cost residency: at C = 4 and 8 it holds 7 and
// 5 wavefronts per SIMD against the immediate build's 8, and decodes the
// 8192 x 28672 stress tensors 24-47% slower, so small chunks always store
// at once.  At C = 16 (4 against 8 per SIMD) the deferred build is used once
// the immediate build's wavefronts would each have at least 24 blocks in
// sequence (a long job, where the spread-out stores pay: the whole model of
// 226 matrices, about 40 blocks per wavefront, decodes 5% faster deferred)
// and its own path is less than twice as long; shorter jobs finish sooner
// with more wavefronts (one Llama-3-8B block, about 10 blocks per
// wavefront, 4% faster immediate).  At C = 32 the immediate build is held
// to 5 per SIMD as well, and the deferred one (4) is 12-27% faster on the
// stress tensors whenever its path is less than twice as long.
template <int C, bool Padded>
dfc_status launch_group(const dfc_batch_item *items, const uint32_t *idx, uint32_t count, uint32_t *status,
                        hipStream_t stream) {
    const uint32_t mode = g_launch.stores.load(std::memory_order_relaxed);
    Plan pd;
    if (mode != DFC_STORES_IMMEDIATE) {
        const dfc_status s = plan_group<C, Padded, true>(items, idx, count, pd);
        if (s != DFC_OK) return s;
        if (mode == DFC_STORES_DEFERRED) return launch_planned<C, Padded, true>(items, pd, status, stream);
    }
    Plan pi;
    const dfc_status s = plan_group<C, Padded, false>(items, idx, count, pi);
    if (s != DFC_OK) return s;
    constexpr uint64_t kMinCrit = C >= 32 ? 0 : 24;
    if (mode == DFC_STORES_AUTO && C >= 16 && pd.crit < 2 * pi.crit && pi.crit >= kMinCrit)
        return launch_planned<C, Padded, true>(items, pd, status, stream);
    return launch_planned<C, Padded, false>(items, pi, status, stream);
}

dfc_status check_item(const dfc_batch_item &it) {
    if (!it.info) return DFC_EINVAL;
    const dfc_info &in = *it.info;
    if (it.n != in.n) return DFC_ESIZE;
    if (in.n == 0) return DFC_OK;
    if (!it.blob_dev || !it.dst_dev) return DFC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(it.blob_dev) & 255u) || (reinterpret_cast<uintptr_t>(it.dst_dev) & 15u) ||
        (reinterpret_cast<uintptr_t>(it.tables_dev) & 15u))
        return DFC_EINVAL;
    if (in.layout == DFC_LAYOUT_ANS) return dfc::ans_check_item(it);
    if (in.layout != DFC_LAYOUT_FLAT && in.layout != DFC_LAYOUT_PADDED) return DFC_EUNSUPPORTED;
    if (in.lanes_per_block != 64) return DFC_EUNSUPPORTED;
    const uint32_t C = in.chunk_bytes;
    if (C != 4 && C != 8 && C != 16 && C != 32) return DFC_EINVAL;
    if (in.lut_bits < 8 || in.lut_bits > 12 || in.min_len < 1) return DFC_EINVAL;
    if (in.max_block_elems > 64u * dfc::ceil_div(8ull * C, in.min_len)) return DFC_EINVAL;
    // Every stream is addressed with 32-bit byte offsets below kNowhere.
    const uint64_t limit = kNowhere - 64u * 1024u;
    if (2 * in.n > limit || in.words_bytes > limit || in.offsets_bytes > limit || in.raw_bytes > limit)
        return DFC_EUNSUPPORTED;
    return DFC_OK;
}

}  // namespace

extern "C" {

dfc_status dfc_set_launch(uint32_t waves_per_group, uint32_t blocks_per_wave, uint32_t stores, uint32_t run_blocks) {
    if (waves_per_group > kMaxWaves) return DFC_EINVAL;
    if (blocks_per_wave > 64) return DFC_EINVAL;
    if (stores > DFC_STORES_IMMEDIATE) return DFC_EINVAL;
    if (run_blocks > 64) return DFC_EINVAL;
    g_launch.waves.store(waves_per_group, std::memory_order_relaxed);
    g_launch.blocks_per_wave.store(blocks_per_wave, std::memory_order_relaxed);
    g_launch.stores.store(stores, std::memory_order_relaxed);
    g_launch.run.store(run_blocks, std::memory_order_relaxed);
    return DFC_OK;
}

dfc_status dfc_derived_tables_bytes(const dfc_info *info, uint64_t *bytes) {
    if (!info || !bytes) return DFC_EINVAL;
    if (info->layout == DFC_LAYOUT_ANS) {
        *bytes = 4ull * dfc::kAnsSlots;
        return DFC_OK;
    }
    if (info->layout != DFC_LAYOUT_FLAT && info->layout != DFC_LAYOUT_PADDED && info->layout != DFC_LAYOUT_PANEL)
        return DFC_EUNSUPPORTED;
    if (info->lut_bits < 8 || info->lut_bits > 12) return DFC_EINVAL;
    *bytes = dfc::tables_bytes(info->lut_bits);
    return DFC_OK;
}

dfc_status dfc_derive_tables(const void *blob_dev, const dfc_info *info, uint32_t threads, void *dst_dev,
                             uint64_t cap, void *stream) {
    uint64_t need = 0;
    const dfc_status s = dfc_derived_tables_bytes(info, &need);
    if (s != DFC_OK) return s;
    if (!blob_dev || !dst_dev || (reinterpret_cast<uintptr_t>(blob_dev) & 255u) ||
        (reinterpret_cast<uintptr_t>(dst_dev) & 15u))
        return DFC_EINVAL;
    if (threads == 0) threads = 1024;
    if (threads % kWave || threads > 1024) return DFC_EINVAL;
    if (cap < need) return DFC_ESIZE;
    if (info->n == 0) return DFC_EINVAL;  // an empty container has no code
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (info->layout == DFC_LAYOUT_ANS) return dfc::ans_derive_tables(blob_dev, *info, threads, dst_dev, st);
    const uint32_t tb = uint32_t(need);
    const size_t lds = size_t(tb) + derive_scratch_bytes(info->lut_bits);
    if (!allow_full_lds(reinterpret_cast<const void *>(&derive_tables_kernel))) return DFC_EHIP;
    derive_tables_kernel<<<dim3(1), dim3(threads), lds, st>>>(
        static_cast<const uint8_t *>(blob_dev) + dfc::hdr::lengths, info->lut_bits, tb, static_cast<uint8_t *>(dst_dev));
    return hipGetLastError() == hipSuccess ? DFC_OK : DFC_EHIP;
}

dfc_status dfc_decode_batch(const dfc_batch_item *items, uint32_t count, uint32_t *status_dev, void *stream) {
    if (count == 0) return DFC_OK;
    if (!items || count > DFC_MAX_BATCH) return DFC_EINVAL;
    for (uint32_t k = 0; k < count; ++k) {
        dfc_status s = check_item(items[k]);
        if (s != DFC_OK) return s;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    static const int sizes[4] = {4, 8, 16, 32};
    {
        uint32_t idx[DFC_MAX_BATCH], m = 0;
        for (uint32_t k = 0; k < count; ++k)
            if (items[k].info->n && items[k].info->layout == DFC_LAYOUT_ANS) idx[m++] = k;
        if (m) {
            dfc_status s = dfc::ans_launch(items, idx, m, status_dev, st);
            if (s != DFC_OK) return s;
        }
    }
    // one launch per (chunk size, layout) present in the batch
    for (int pad = 0; pad < 2; ++pad) {
        const uint32_t layout = pad ? DFC_LAYOUT_PADDED : DFC_LAYOUT_FLAT;
        for (int c : sizes) {
            uint32_t idx[DFC_MAX_BATCH], m = 0;
            for (uint32_t k = 0; k < count; ++k) {
                const dfc_info &in = *items[k].info;
                if (in.n && in.chunk_bytes == uint32_t(c) && in.layout == layout) idx[m++] = k;
            }
            if (!m) continue;
            dfc_status s = DFC_OK;
            switch (c * 2 + pad) {
                case 8: s = launch_group<4, false>(items, idx, m, status_dev, st); break;
                case 9: s = launch_group<4, true>(items, idx, m, status_dev, st); break;
                case 16: s = launch_group<8, false>(items, idx, m, status_dev, st); break;
                case 17: s = launch_group<8, true>(items, idx, m, status_dev, st); break;
                case 32: s = launch_group<16, false>(items, idx, m, status_dev, st); break;
                case 33: s = launch_group<16, true>(items, idx, m, status_dev, st); break;
                case 64: s = launch_group<32, false>(items, idx, m, status_dev, st); break;
                default: s = launch_group<32, true>(items, idx, m, status_dev, st); break;
            }
            if (s != DFC_OK) return s;
        }
    }
    return DFC_OK;
}

dfc_status dfc_decode(const void *blob_dev, const dfc_info *info, const void *tables_dev, uint16_t *dst_dev,
                      uint64_t n, uint32_t *status_dev, void *stream) {
    dfc_batch_item it;
    it.blob_dev = blob_dev;
    it.info = info;
    it.tables_dev = tables_dev;
    it.dst_dev = dst_dev;
    it.n = n;
    return dfc_decode_batch(&it, 1, status_dev, stream);
}

}  // extern "C"
