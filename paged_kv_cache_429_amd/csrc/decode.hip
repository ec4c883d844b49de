// Paged decode attention for gfx950.
//
// What is computed ("KV cache, continuous batching and paged attention",
// section "Paged attention": the attention kernel follows the block table):
// for every sequence s and query head h,
//     o[s,h] = softmax(q[s,h] . K_s^T / sqrt(d)) V_s
// where K_s / V_s are the context_lens[s] cached tokens of KV head h / G,
// found through the sequence's block table.
//
// Work decomposition. One workgroup (4 waves) per (sequence, KV head,
// context partition), partitions in descending order; the KV head is the
// fastest-varying index, so with 8 KV heads each head's workgroups land on
// one XCD (workgroups are dealt to the 8 XCDs round-robin). A partition is `pb` consecutive logical blocks; the
// waves take pairs of blocks round-robin. All G query heads of the KV head
// are processed together, so each K/V tile is read from HBM once per KV head
// (GQA batching, "KV cache, GQA, paging and continuous batching", section
// "What it is"). Waves keep an online softmax (running max m, running sum l,
// unnormalised accumulator), merge through LDS, and either write the output
// (single partition) or a partial (m, l, acc) to the workspace; the last
// workgroup of a (sequence, KV head) to finish merges the partials with a
// log-sum-exp reduction in partition order and re-arms its arrival counter,
// so one launch does the whole step.
//
// MFMA formulation (bf16 / int8 / int4 / fp8 KV). Per pair of blocks:
//   S^T[32 tok x 16 col] = K[tok x d] * Q^T[d x col]   (2 x D/32 MFMA 16x16x32)
//   O^T[d x col]        += V^T[d x 32 tok] * P^T[32 tok x col] (D/16 MFMA)
// The 16 columns are the G query heads of the KV head (zero-padded). The K
// tile is stored in 16-byte chunks of consecutive dims (slot-minor), so a
// lane's K operand is one 16-byte load and a wave's load instruction reads a
// contiguous 1 KiB. The V tile is stored transposed (a row is the 16 tokens
// of one dim), and the P.V product's k index gives lane group q the 8
// consecutive tokens 8 (q % 2) .. + 7 of block q / 2: a lane's V operand is
// one contiguous half row (16 B for bf16), and the probabilities are
// regrouped from the S^T accumulator layout by two cross-row lane swaps.
//
// fp32 KV uses a plain VALU path with the same decomposition and epilogue.
#include "pa_attn.h"

namespace pa {

// Waves per SIMD the register budget is sized for: the bf16 loop fits three
// (<= 168 VGPRs); the int4 loop, with two pairs in flight, needs more (int8
// and fp8 stay under 168 and run at three anyway).
template <int FMT>
constexpr int decode_waves_per_eu() {
    return FMT == FMT_BF16 ? 3 : 2;
}

template <int D, int FMT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<FMT>())))
void decode_kernel(DecodeParams p) {
    // the waves' states; once merged, the partial-merge scratch
    constexpr size_t kLds = sizeof(WaveState<D>) > kMergeFloats * sizeof(float) ? sizeof(WaveState<D>)
                                                                               : kMergeFloats * sizeof(float);
    constexpr int kCap = (int)(kLds / sizeof(float));
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
    WaveState<D>& st = *reinterpret_cast<WaveState<D>*>(smem);
    float* const scratch = reinterpret_cast<float*>(smem);
    constexpr bool F32OUT = (FMT == FMT_F32);
    Unit u;
    const int unit = blockIdx.x;
    u.kvh = unit % p.n_kv;
    const int rest = unit / p.n_kv;
    // Highest partitions first, partition 0 of every sequence last: the
    // last round of workgroups then holds whole short sequences and full
    // first partitions, of similar size, instead of a random mix (the
    // order changes nothing but when a unit runs). With the prefix pass,
    // partition 0 of every sequence comes first instead: the run usually
    // leaves a sequence one short partition, so the units left without
    // blocks fall at the end of the launch, where they exit while the last
    // real units run.
    if (p.prefix_ts > 0) {
        u.s = rest % p.num_seqs;
        u.part = rest / p.num_seqs;
    } else {
        u.s = rest % p.num_seqs;
        u.part = p.pmax - 1 - rest / p.num_seqs;
    }
    // Without a prefix pass or a window the partition starts at block
    // part * pb whatever the length, so its block ids are fetched together
    // with the length (entries past the sequence's end are never used)
    // instead of one memory round trip later.
    const int32_t* trow = p.tables + (size_t)u.s * p.max_blocks;
    const bool ids_early = FMT != FMT_F32 && p.prefix_ts == 0 && p.window == 0;
    int wave_ids = 0;
    if (ids_early) {  // entries as stored; checked once the partition's extent is known
        const int first = u.part * p.pb;  // < blocks of a sequence at ctx_cap <= max_blocks
        wave_ids = load_wave_ids_raw(trow, first, min(p.max_blocks - first, kMaxPartitionBlocks));
    }
    u.ctx = min(p.ctx[u.s], p.ctx_cap);
    if (u.ctx <= 0) {
        if (u.part == 0) {
            for (int idx = threadIdx.x; idx < p.group * D; idx += kThreads)
                store_out<D, F32OUT>(p, ((size_t)u.s * p.n_heads + u.kvh * p.group) * D + idx, 0.f);
        }
        return;
    }
    u.nblk = (u.ctx + kBlock - 1) / kBlock;
    // blocks [0, run) were attended by the prefix pass (run < nblk); with a
    // sliding window (never together with the prefix pass) the blocks
    // before the one holding the window's first token are skipped
    const int run = p.prefix_ts > 0 ? p.plan[u.s / p.prefix_ts] : 0;
    u.lo = p.window > 0 ? max(0, u.ctx - p.window) : 0;
    const int b0 = p.window > 0 ? u.lo / kBlock : run;
    u.slot0 = prefix_parts(run, p.kpmax);
    u.nparts = num_parts(u.nblk - b0, p.pb);
    if (u.part >= u.nparts) return;
    u.b_begin = b0 + u.part * p.pb;
    u.b_end = b0 + part_end(u.nblk - b0, p.pb, u.part, u.nparts);
    if constexpr (FMT != FMT_F32) {
        // A group of share_n sequences that shares this partition's first
        // pair is computed by the workgroup of its first sequence, for all
        // of them; the others' workgroups have nothing to do.
        if (p.share_n > 0 && b0 == 0) {
            const int grp = u.s / p.share_n;
            const int s0 = grp * p.share_n;
            if (s0 + p.share_n <= p.num_seqs && group_shares(p, s0, u.part)) {
                if (u.s == s0) {
                    const int gunit = (grp * p.pmax + u.part) * p.n_kv + u.kvh;
                    if (p.share_n == 2) {
                        shared_unit<D, FMT, 1, 2, F32OUT>(p, gunit, st, scratch, kCap);
                    } else {
                        shared_unit<D, FMT, 1, 4, F32OUT>(p, gunit, st, scratch, kCap);
                    }
                }
                return;
            }
        }
    }

    if constexpr (FMT == FMT_F32) {
        __shared__ float qs[16 * D];
        const float* qg = reinterpret_cast<const float*>(p.q) + ((size_t)u.s * p.n_heads + u.kvh * p.group) * D;
        for (int idx = threadIdx.x; idx < p.group * D; idx += kThreads) qs[idx] = qg[idx];
        __syncthreads();
        f32_wave<D>(p, u, trow, st, qs);
    } else {
        if (ids_early) {
            wave_ids = check_wave_ids(wave_ids, p.tables, trow, u.b_begin, u.b_end - u.b_begin, p.num_blocks);
        } else {
            wave_ids = load_wave_ids(p.tables, trow, u.b_begin, u.b_end - u.b_begin, p.num_blocks);
        }
        mfma_wave<D, FMT>(p, u, wave_ids, st);
    }
    epilogue<D, F32OUT>(p, u, st, scratch, kCap);
}

hipError_t take_bad_id_decode(BadIdRecord* out) {
    const BadIdRecord zero{};
    hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_bad_ids), sizeof(BadIdRecord), 0, hipMemcpyDeviceToHost);
    if (e == hipSuccess && out->flag)
        e = hipMemcpyToSymbol(HIP_SYMBOL(g_bad_ids), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
    return e;
}

// Workspace: a fixed-size region of arrival words at offset 0, then the
// partial accumulators and (max, sum) pairs. Because the counter region
// never moves or shrinks, calls of any shape can share one workspace:
// partial data never lands on the arrival words, and those are tagged with
// each call's epoch, so no call depends on what an earlier one left there.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The prefix pass adds kpmax partial slots per (sequence, query head) and
// one plan entry per tile (num_seqs entries bound the tile count).
size_t decode_workspace_bytes(int num_seqs, int n_heads, int n_kv, int d, int pmax, int kpmax) {
    (void)n_kv;
    if (pmax <= 1 && kpmax == 0) return 0;  // nothing is split: no partials
    const size_t rows = (size_t)num_seqs * n_heads * (pmax + kpmax);
    const size_t plan = kpmax > 0 ? align256((size_t)num_seqs * sizeof(int)) : 0;
    return kCounterBytes + align256(rows * d * sizeof(float)) + align256(rows * 2 * sizeof(float)) + plan;
}

void decode_workspace_carve(void* ws, int num_seqs, int n_heads, int n_kv, int d, int pmax, int kpmax,
                            float** part_acc, float** part_ml, unsigned long long** counters, int** plan) {
    (void)n_kv;
    const size_t rows = (size_t)num_seqs * n_heads * (pmax + kpmax);
    char* b = static_cast<char*>(ws);
    *counters = reinterpret_cast<unsigned long long*>(b);
    b += kCounterBytes;
    *part_acc = reinterpret_cast<float*>(b);
    b += align256(rows * d * sizeof(float));
    *part_ml = reinterpret_cast<float*>(b);
    b += align256(rows * 2 * sizeof(float));
    *plan = kpmax > 0 ? reinterpret_cast<int*>(b) : nullptr;
}

template <int D, int FMT>
static hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
    const size_t grid = (size_t)p.num_seqs * p.pmax * p.n_kv;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffffu) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_kernel<D, FMT>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int d, int fmt, hipStream_t stream) {
    if (d == 128) {
        switch (fmt) {
            case FMT_F32: return launch_t<128, FMT_F32>(p, stream);
            case FMT_BF16: return launch_t<128, FMT_BF16>(p, stream);
            case FMT_I8: return launch_t<128, FMT_I8>(p, stream);
            case FMT_I4: return launch_t<128, FMT_I4>(p, stream);
            case FMT_F8: return launch_t<128, FMT_F8>(p, stream);
        }
    } else if (d == 64) {
        switch (fmt) {
            case FMT_F32: return launch_t<64, FMT_F32>(p, stream);
            case FMT_BF16: return launch_t<64, FMT_BF16>(p, stream);
            case FMT_I8: return launch_t<64, FMT_I8>(p, stream);
            case FMT_I4: return launch_t<64, FMT_I4>(p, stream);
            case FMT_F8: return launch_t<64, FMT_F8>(p, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
