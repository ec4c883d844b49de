// Host-side block manager and scheduler step (include/pa_block_manager.h).
//
// Paging, sharing and prefix reuse follow "KV cache, GQA, paging and
// continuous batching", sections "PagedAttention: why fragmentation was
// eating most of the rest" (block table, on-demand blocks, copy-on-write at
// divergence), "Prefix caching: the biggest single lever most teams have"
// (a prefix match over whole blocks) and "The scheduler, and preemption"
// (admission bounded by free blocks, the newest sequence preempted when
// memory runs out). The rules the pages leave open are listed in the header.
#include "../../include/pa_block_manager.h"

#include <algorithm>
#include <array>
#include <cstdint>
#include <deque>
#include <map>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

namespace {

constexpr int kBlock = PA_BLOCK_SIZE;
using BlockToks = std::array<int64_t, kBlock>;

// Prefix cache as a trie over whole blocks: the node reached from the root
// by the token contents of blocks 0..i of a prompt stands for that exact
// prefix, and holds the physical block cached for its last block (-1 when
// none is). Lookups compare token contents exactly, so two different
// prefixes never share an entry.
struct Node {
    Node* parent = nullptr;
    BlockToks toks{};
    std::map<BlockToks, Node*> kids;
    int32_t block = -1;
};

BlockToks block_toks(const int64_t* t) {
    BlockToks b;
    std::copy(t, t + kBlock, b.begin());
    return b;
}

struct Seq {
    std::vector<int32_t> table;
    int n = 0;
};

}  // namespace

struct pa_block_manager {
    int num_blocks = 0;
    bool prefix_cache = false;
    std::deque<int32_t> free_q;
    // evictable cached blocks, least recently released first: a doubly
    // linked list threaded through prev/next (-1 ends), head = oldest
    std::vector<int32_t> prev, next;
    std::vector<uint8_t> in_lru;
    int32_t head = -1, tail = -1;
    int n_evictable = 0;
    std::vector<int32_t> ref;
    Node root;
    std::vector<Node*> node_of;   // trie node of a cached block, else nullptr
    std::vector<Node*> evicted;   // nodes that lost their block in this operation
    std::unordered_map<int64_t, Seq> seqs;

    ~pa_block_manager() { free_kids(&root); }
    static void free_kids(Node* n) {
        for (auto& kv : n->kids) {
            free_kids(kv.second);
            delete kv.second;
        }
        n->kids.clear();
    }

    int num_free() const { return (int)free_q.size() + n_evictable; }

    void lru_push(int32_t b) {
        prev[b] = tail;
        next[b] = -1;
        if (tail >= 0) next[tail] = b; else head = b;
        tail = b;
        in_lru[b] = 1;
        ++n_evictable;
    }
    void lru_remove(int32_t b) {
        if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
        if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
        prev[b] = next[b] = -1;
        in_lru[b] = 0;
        --n_evictable;
    }
    // caller has checked num_free() >= 1
    int32_t take() {
        int32_t b;
        if (!free_q.empty()) {
            b = free_q.front();
            free_q.pop_front();
        } else {
            b = head;
            lru_remove(b);
            Node* n = node_of[b];
            n->block = -1;
            node_of[b] = nullptr;
            evicted.push_back(n);
        }
        ref[b] = 1;
        return b;
    }
    void drop(int32_t b) {
        if (--ref[b] == 0) {
            if (node_of[b]) lru_push(b); else free_q.push_back(b);
        }
    }
    // The child of n for block content t, created if missing.
    Node* child(Node* n, const BlockToks& t) {
        auto it = n->kids.find(t);
        if (it != n->kids.end()) return it->second;
        Node* c = new Node;
        c->parent = n;
        c->toks = t;
        n->kids.emplace(t, c);
        return c;
    }
    // End of an operation: drop the trie nodes that now hold no block and
    // lead to none (deferred so that no node goes away while an operation
    // holds it).
    // (A work set, not a walk up from each node: two evicted nodes may lie
    // on one path, and removing the lower one can remove the upper one.)
    void prune() {
        std::set<Node*> work(evicted.begin(), evicted.end());
        evicted.clear();
        while (!work.empty()) {
            Node* n = *work.begin();
            work.erase(work.begin());
            if (n == &root || n->block >= 0 || !n->kids.empty()) continue;
            Node* p = n->parent;
            p->kids.erase(n->toks);
            delete n;
            work.insert(p);
        }
    }
};

extern "C" {

pa_block_manager* pa_bm_create(int num_blocks, int prefix_cache) {
    if (num_blocks <= 0 || (prefix_cache != 0 && prefix_cache != 1)) return nullptr;
    pa_block_manager* bm = new (std::nothrow) pa_block_manager;
    if (!bm) return nullptr;
    try {
        bm->num_blocks = num_blocks;
        bm->prefix_cache = prefix_cache != 0;
        for (int32_t b = 0; b < num_blocks; ++b) bm->free_q.push_back(b);
        bm->prev.assign(num_blocks, -1);
        bm->next.assign(num_blocks, -1);
        bm->in_lru.assign(num_blocks, 0);
        bm->ref.assign(num_blocks, 0);
        bm->node_of.assign(num_blocks, nullptr);
    } catch (...) {
        delete bm;
        return nullptr;
    }
    return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int pa_bm_num_free(const pa_block_manager* bm) { return bm ? bm->num_free() : PA_ERR_INVALID_ARG; }

int pa_bm_ref_count(const pa_block_manager* bm, int block) {
    if (!bm || block < 0 || block >= bm->num_blocks) return -1;
    return bm->ref[block];
}

int pa_bm_add(pa_block_manager* bm, int64_t seq, const int64_t* tokens, int n_tokens, int* cached_tokens) {
    if (!bm || n_tokens < 0 || (n_tokens > 0 && !tokens)) return PA_ERR_INVALID_ARG;
    if (bm->seqs.count(seq)) return PA_ERR_NO_SEQUENCE;
    try {
        const int nblk = (n_tokens + kBlock - 1) / kBlock;
        const int full = n_tokens / kBlock;
        // the longest cached prefix of whole blocks: walk the trie while each
        // block's node holds a cached block
        std::vector<int32_t> hits;
        if (bm->prefix_cache) {
            const Node* cur = &bm->root;
            for (int i = 0; i < full; ++i) {
                auto it = cur->kids.find(block_toks(tokens + (size_t)i * kBlock));
                if (it == cur->kids.end() || it->second->block < 0) break;
                cur = it->second;
                hits.push_back(cur->block);
            }
        }
        int revived = 0;
        for (int32_t b : hits) revived += bm->ref[b] == 0;
        const int need = nblk - (int)hits.size();
        if (need > bm->num_free() - revived) return PA_ERR_NO_BLOCKS;
        Seq s;
        s.table.reserve(nblk);
        s.n = n_tokens;
        Node* cur = &bm->root;
        for (size_t i = 0; i < hits.size(); ++i) {
            const int32_t b = hits[i];
            if (bm->ref[b] == 0) bm->lru_remove(b);
            ++bm->ref[b];
            s.table.push_back(b);
            cur = bm->node_of[b];
        }
        for (int i = (int)hits.size(); i < nblk; ++i) {
            const int32_t b = bm->take();
            s.table.push_back(b);
            // a full prompt block is cached under its prefix unless a block
            // is already cached there
            if (bm->prefix_cache && i < full) {
                cur = bm->child(cur, block_toks(tokens + (size_t)i * kBlock));
                if (cur->block < 0) {
                    cur->block = b;
                    bm->node_of[b] = cur;
                }
            }
        }
        bm->seqs.emplace(seq, std::move(s));
        bm->prune();
        if (cached_tokens) *cached_tokens = (int)hits.size() * kBlock;
        return PA_OK;
    } catch (...) {
        bm->prune();
        return PA_ERR_INVALID_ARG;
    }
}

int pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t* cow_src, int32_t* cow_dst) {
    if (!bm || !cow_src || !cow_dst) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
    Seq& s = it->second;
    *cow_src = *cow_dst = -1;
    try {
        if (s.n % kBlock == 0) {
            if (bm->num_free() < 1) return PA_ERR_NO_BLOCKS;
            s.table.reserve(s.table.size() + 1);
            s.table.push_back(bm->take());
        } else if (bm->ref[s.table.back()] > 1) {
            if (bm->num_free() < 1) return PA_ERR_NO_BLOCKS;
            const int32_t src = s.table.back();
            const int32_t dst = bm->take();
            bm->drop(src);
            s.table.back() = dst;
            *cow_src = src;
            *cow_dst = dst;
        }
    } catch (...) {
        bm->prune();
        return PA_ERR_INVALID_ARG;
    }
    bm->prune();
    ++s.n;
    return PA_OK;
}

int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child) {
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end() || bm->seqs.count(child)) return PA_ERR_NO_SEQUENCE;
    try {
        Seq c = it->second;
        for (int32_t b : c.table) ++bm->ref[b];
        bm->seqs.emplace(child, std::move(c));
    } catch (...) {
        return PA_ERR_INVALID_ARG;
    }
    return PA_OK;
}

int pa_bm_release(pa_block_manager* bm, int64_t seq) {
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
    const std::vector<int32_t>& t = it->second.table;
    for (auto b = t.rbegin(); b != t.rend(); ++b) bm->drop(*b);
    bm->seqs.erase(it);
    return PA_OK;
}

int pa_bm_num_tokens(const pa_block_manager* bm, int64_t seq) {
    if (!bm) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq);
    return it == bm->seqs.end() ? PA_ERR_NO_SEQUENCE : it->second.n;
}

int pa_bm_table(const pa_block_manager* bm, int64_t seq, int32_t* row, int max_blocks) {
    if (!bm || max_blocks < 0 || (max_blocks > 0 && !row)) return PA_ERR_INVALID_ARG;
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PA_ERR_NO_SEQUENCE;
    const std::vector<int32_t>& t = it->second.table;
    std::copy(t.begin(), t.begin() + std::min<size_t>(t.size(), (size_t)max_blocks), row);
    return (int)t.size();
}

}  // extern "C"

struct pa_scheduler {
    pa_block_manager* bm = nullptr;
    std::deque<int64_t> waiting;
    std::vector<int64_t> running;  // oldest first
    std::unordered_map<int64_t, std::vector<int64_t>> tokens;
};

extern "C" {

pa_scheduler* pa_sched_create(pa_block_manager* bm) {
    if (!bm) return nullptr;
    pa_scheduler* s = new (std::nothrow) pa_scheduler;
    if (s) s->bm = bm;
    return s;
}

void pa_sched_destroy(pa_scheduler* s) { delete s; }

int pa_sched_submit(pa_scheduler* s, int64_t seq, const int64_t* prompt, int n_prompt) {
    if (!s || n_prompt < 0 || (n_prompt > 0 && !prompt)) return PA_ERR_INVALID_ARG;
    if (s->tokens.count(seq)) return PA_ERR_NO_SEQUENCE;
    try {
        s->tokens.emplace(seq, std::vector<int64_t>(prompt, prompt + n_prompt));
        s->waiting.push_back(seq);
    } catch (...) {
        return PA_ERR_INVALID_ARG;
    }
    return PA_OK;
}

int pa_sched_num_live(const pa_scheduler* s) { return s ? (int)s->tokens.size() : PA_ERR_INVALID_ARG; }

int pa_sched_step(pa_scheduler* s, int cap, int64_t* running, int* n_running, int64_t* preempted, int* n_preempted,
                  int32_t* cow, int* n_cow, int* n_stalled) {
    if (!s || !running || !n_running || !preempted || !n_preempted || !cow || !n_cow || !n_stalled)
        return PA_ERR_INVALID_ARG;
    if (cap < (int)s->tokens.size()) return PA_ERR_INVALID_ARG;
    pa_block_manager* bm = s->bm;
    while (!s->waiting.empty()) {
        const int64_t q = s->waiting.front();
        const std::vector<int64_t>& t = s->tokens[q];
        const int st = pa_bm_add(bm, q, t.data(), (int)t.size(), nullptr);
        if (st == PA_ERR_NO_BLOCKS) break;
        if (st != PA_OK) return st;
        s->waiting.pop_front();
        s->running.push_back(q);
    }
    int np = 0, nc = 0, nr = 0, stalled = 0;
    int64_t stalled_id = 0;
    size_t i = 0;
    while (i < s->running.size()) {
        const int64_t q = s->running[i];
        int32_t src, dst;
        const int st = pa_bm_append(bm, q, &src, &dst);
        if (st == PA_ERR_NO_BLOCKS) {
            if (s->running.size() == 1) {
                stalled = 1;
                stalled_id = q;
                ++i;
                continue;
            }
            const int64_t victim = s->running.back();
            s->running.pop_back();
            pa_bm_release(bm, victim);
            s->waiting.push_front(victim);
            preempted[np++] = victim;
            continue;
        }
        if (st != PA_OK) return st;
        if (src >= 0) {
            cow[2 * nc] = src;
            cow[2 * nc + 1] = dst;
            ++nc;
        }
        ++i;
    }
    for (int64_t q : s->running) {
        if (!(stalled && q == stalled_id)) running[nr++] = q;
    }
    *n_running = nr;
    *n_preempted = np;
    *n_cow = nc;
    *n_stalled = stalled;
    return PA_OK;
}

int pa_sched_record(pa_scheduler* s, int64_t seq, int64_t token) {
    if (!s) return PA_ERR_INVALID_ARG;
    auto it = s->tokens.find(seq);
    if (it == s->tokens.end() || std::find(s->running.begin(), s->running.end(), seq) == s->running.end())
        return PA_ERR_NO_SEQUENCE;
    try {
        it->second.push_back(token);
    } catch (...) {
        return PA_ERR_INVALID_ARG;
    }
    return PA_OK;
}

int pa_sched_finish(pa_scheduler* s, int64_t seq) {
    if (!s) return PA_ERR_INVALID_ARG;
    auto r = std::find(s->running.begin(), s->running.end(), seq);
    if (r == s->running.end()) return PA_ERR_NO_SEQUENCE;
    s->running.erase(r);
    s->tokens.erase(seq);
    return pa_bm_release(s->bm, seq);
}

}  // extern "C"
