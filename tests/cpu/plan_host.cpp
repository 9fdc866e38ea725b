// Host build of the prefill's chunk plan (plan_sequences, the function the
// GPU plan kernel runs), one thread per lane of the 1024-thread workgroup and
// a barrier for each workgroup barrier.  It checks the plan's memory bounds:
// the segment and chunk tables sit between guard zones that must come out
// untouched, whatever cu_seqlens holds.
//
// stdin:  nseq seqlen total chunk max_chunks, then nseq+1 cu_seqlens values
//         (seqlen >= 0 and no values: uniform rows)
// stdout: "error n_chunks guards_ok", then one line "first count" per
//         sequence, then one line "start len seq" per chunk in the table
#include <pthread.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "plan_body.h"

namespace {

constexpr int NT = 1024;
constexpr int GUARD = 4096;  // entries of each guard zone
constexpr unsigned char FILL = 0xA5;

struct HostCtx {
    int64_t* scan;
    std::atomic<int32_t>* bad;
    std::atomic<int32_t>* err;
    pthread_barrier_t* bar;
    int t;
    int tid() const { return t; }
    void sync() const { pthread_barrier_wait(bar); }
};

template <class T>
bool untouched(const std::vector<T>& v, size_t n_inner) {
    const unsigned char* p = reinterpret_cast<const unsigned char*>(v.data());
    const size_t g = GUARD * sizeof(T), inner = n_inner * sizeof(T);
    for (size_t i = 0; i < g; ++i)
        if (p[i] != FILL || p[g + inner + i] != FILL) return false;
    return true;
}

}  // namespace

int main() {
    long long nseq_l, seqlen, total, chunk_l, maxc_l;
    if (scanf("%lld %lld %lld %lld %lld", &nseq_l, &seqlen, &total, &chunk_l, &maxc_l) != 5)
        return 2;
    const int nseq = (int)nseq_l, chunk = (int)chunk_l, max_chunks = (int)maxc_l;
    std::vector<int32_t> cu;
    if (seqlen < 0) {
        cu.resize(nseq + 1);
        for (int i = 0; i <= nseq; ++i) {
            long long x;
            if (scanf("%lld", &x) != 1) return 2;
            cu[i] = (int32_t)x;
        }
    }
    la::PlanHeader hdr;
    std::memset(&hdr, 0, sizeof(hdr));
    std::vector<la::SegEntry> segs(nseq + 2 * GUARD);
    std::vector<la::ChunkEntry> chunks(max_chunks + 2 * GUARD);
    std::memset(segs.data(), FILL, segs.size() * sizeof(la::SegEntry));
    std::memset(chunks.data(), FILL, chunks.size() * sizeof(la::ChunkEntry));
    std::vector<int64_t> scan(NT);
    std::atomic<int32_t> bad{0}, err{0};
    pthread_barrier_t bar;
    pthread_barrier_init(&bar, nullptr, NT);
    std::vector<std::thread> th;
    for (int t = 0; t < NT; ++t)
        th.emplace_back([&, t] {
            HostCtx x{scan.data(), &bad, &err, &bar, t};
            la::plan_sequences<NT>(x, cu.empty() ? nullptr : cu.data(), nseq,
                                   seqlen < 0 ? 0 : seqlen, total, chunk, max_chunks, &hdr,
                                   segs.data() + GUARD, chunks.data() + GUARD);
        });
    for (auto& t : th) t.join();
    pthread_barrier_destroy(&bar);
    const bool ok = untouched(segs, nseq) && untouched(chunks, max_chunks);
    printf("%d %d %d\n", hdr.error, hdr.n_chunks, ok ? 1 : 0);
    for (int s = 0; s < nseq; ++s) printf("%d %d\n", segs[GUARD + s].first, segs[GUARD + s].count);
    for (int c = 0; c < hdr.n_chunks && c < max_chunks; ++c) {
        const la::ChunkEntry& e = chunks[GUARD + c];
        printf("%lld %d %d\n", (long long)e.start, e.len, e.seg);
    }
    return 0;
}
