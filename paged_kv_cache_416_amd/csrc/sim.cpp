// Continuous-batching memory simulator: the memory side of iteration-level scheduling (lesson
// note "Week 22 Day 2", section 4) under the paged scheme -- this library's block pool, with
// all-or-nothing eviction of the newest request when a decode step runs short (slide 15) --
// and under contiguous reservations placed first-fit in one linear range (lesson note section 1;
// slide 6: reservation, internal and external fragmentation). Host only.
//
// One step, in this order: arrivals join the queue tail; every running request appends one
// token (paged: one batched pkv_seq_append; on PKV_ENOMEM the newest running request is freed
// and put back at the queue head, and the append is tried again); requests that reached their
// output length are freed; the queue head is admitted while it fits and the batch is below
// max_batch, its prefill writing its prompt plus the tokens it generated before any eviction
// (recompute); then one trace row is written.
#include <deque>
#include <iterator>
#include <map>
#include <vector>

#include "common.h"

namespace pkv {
namespace {

enum Field {
    kStep, kRunning, kWaiting, kUsed, kHeld, kFree, kLargestFree, kAdmitted, kPreempted, kFinished, kDecoded,
    kBlockedNeed, kFinalSum, kFields
};
static_assert(kFields == PKV_SIM_FIELDS, "trace row layout");

// The memory side of one scheme; the step loop below is shared.
struct Memory {
    virtual ~Memory() = default;
    virtual int admit(int32_t r, int64_t tokens, bool *ok) = 0;  // prefill of `tokens` tokens
    virtual int grow(const std::vector<int32_t> &running, bool *ok) = 0;  // one token each
    virtual int release(int32_t r) = 0;
    virtual int64_t need(int32_t r, int64_t tokens) const = 0;  // slots an admission asks for
    virtual int64_t held() const = 0;
    virtual int64_t largest_free() const = 0;
};

class PagedMemory final : public Memory {
  public:
    PagedMemory(pkv_pool *pool, int32_t B, int32_t N, int32_t watermark)
        : pool_(pool), B_(B), N_(N), watermark_(watermark) {}
    int admit(int32_t r, int64_t tokens, bool *ok) override {
        *ok = false;
        if (pkv_pool_num_free(pool_) < ceil_div(tokens, B_) + watermark_) return PKV_OK;
        int rc = pkv_seq_add(pool_, r);
        if (rc) return rc;
        const int64_t id = r;
        const int32_t n = static_cast<int32_t>(tokens);
        slots_.resize(static_cast<size_t>(tokens));
        rc = pkv_seq_append(pool_, &id, &n, 1, slots_.data(), nullptr, 0, nullptr);
        if (rc) return rc;  // the free-block check above makes PKV_ENOMEM impossible here
        *ok = true;
        return PKV_OK;
    }
    int grow(const std::vector<int32_t> &running, bool *ok) override {
        ids_.assign(running.begin(), running.end());
        ones_.assign(running.size(), 1);
        slots_.resize(running.size());
        const int rc = pkv_seq_append(pool_, ids_.data(), ones_.data(), static_cast<int32_t>(running.size()),
                                      slots_.data(), nullptr, 0, nullptr);
        *ok = rc == PKV_OK;
        return rc == PKV_ENOMEM ? PKV_OK : rc;
    }
    int release(int32_t r) override { return pkv_seq_free(pool_, r); }
    int64_t need(int32_t, int64_t tokens) const override { return ceil_div(tokens, B_) * B_; }
    int64_t held() const override { return static_cast<int64_t>(N_ - pkv_pool_num_free(pool_)) * B_; }
    int64_t largest_free() const override { return static_cast<int64_t>(pkv_pool_num_free(pool_)) * B_; }

  private:
    pkv_pool *pool_;
    int64_t B_;
    int32_t N_, watermark_;
    std::vector<int64_t> ids_, slots_;
    std::vector<int32_t> ones_;
};

class ContiguousMemory final : public Memory {
  public:
    ContiguousMemory(int64_t capacity, const int32_t *reserve) : reserve_(reserve) {
        holes_[0] = capacity;
    }
    int admit(int32_t r, int64_t, bool *ok) override {
        const int64_t R = reserve_[r];
        *ok = false;
        for (auto it = holes_.begin(); it != holes_.end(); ++it) {  // first fit: lowest address
            if (it->second < R) continue;
            const int64_t off = it->first, size = it->second;
            holes_.erase(it);
            if (size > R) holes_[off + R] = size - R;
            where_[r] = off;
            held_ += R;
            *ok = true;
            break;
        }
        return PKV_OK;
    }
    int grow(const std::vector<int32_t> &, bool *ok) override {
        *ok = true;  // the reservation covers the request's final length
        return PKV_OK;
    }
    int release(int32_t r) override {
        const auto w = where_.find(r);
        int64_t off = w->second, size = reserve_[r];
        where_.erase(w);
        held_ -= size;
        auto next = holes_.lower_bound(off);
        if (next != holes_.end() && off + size == next->first) {  // merge with the hole above
            size += next->second;
            next = holes_.erase(next);
        }
        if (next != holes_.begin()) {  // and with the hole below
            auto prev = std::prev(next);
            if (prev->first + prev->second == off) {
                prev->second += size;
                return PKV_OK;
            }
        }
        holes_[off] = size;
        return PKV_OK;
    }
    int64_t need(int32_t r, int64_t) const override { return reserve_[r]; }
    int64_t held() const override { return held_; }
    int64_t largest_free() const override {
        int64_t m = 0;
        for (const auto &h : holes_) m = h.second > m ? h.second : m;
        return m;
    }

  private:
    const int32_t *reserve_;
    std::map<int64_t, int64_t> holes_;  // offset -> size, disjoint and never adjacent
    std::map<int32_t, int64_t> where_;  // request -> offset of its reservation
    int64_t held_ = 0;
};

int check_requests(const char *fn, const int32_t *arrival, const int32_t *prompt, const int32_t *output,
                   int32_t n) {
    if (n < 0 || (n > 0 && (!arrival || !prompt || !output)))
        return fail(PKV_EINVAL, "%s: bad request arrays", fn);
    for (int32_t i = 0; i < n; ++i) {
        if (arrival[i] < 0 || (i > 0 && arrival[i] < arrival[i - 1]))
            return fail(PKV_EINVAL, "%s: arrival steps must be >= 0 and non-decreasing (request %d)", fn, i);
        if (prompt[i] < 1 || output[i] < 1)
            return fail(PKV_EINVAL, "%s: request %d has prompt %d, output %d (both must be >= 1)", fn, i, prompt[i],
                        output[i]);
        if (static_cast<int64_t>(prompt[i]) + output[i] > INT32_MAX)
            return fail(PKV_EINVAL, "%s: request %d is too long", fn, i);
    }
    return PKV_OK;
}

int run(const char *fn, Memory &mem, int64_t capacity, int32_t max_batch, const int32_t *arrival,
        const int32_t *prompt, const int32_t *output, int32_t n, int64_t max_steps, int64_t *trace,
        int64_t *n_steps_out, int64_t *finish) {
    std::vector<int32_t> gen(static_cast<size_t>(n), 0);
    for (int32_t i = 0; i < n; ++i) finish[i] = -1;
    std::deque<int32_t> waiting;
    std::vector<int32_t> running, kept;  // admission order: the back is the newest
    int32_t next = 0;
    for (int64_t t = 0;; ++t) {
        if (t >= max_steps)
            return fail(PKV_EINVAL, "%s: requests still running or waiting after max_steps = %lld", fn,
                        static_cast<long long>(max_steps));
        while (next < n && arrival[next] == t) waiting.push_back(next++);
        int64_t preempted = 0;
        while (!running.empty()) {
            bool ok = false;
            int rc = mem.grow(running, &ok);
            if (rc) return rc;
            if (ok) break;
            const int32_t victim = running.back();  // slide 15: the newest request leaves whole
            running.pop_back();
            rc = mem.release(victim);
            if (rc) return rc;
            waiting.push_front(victim);
            ++preempted;
        }
        const int64_t decoded = static_cast<int64_t>(running.size());
        int64_t finished = 0;
        kept.clear();
        for (const int32_t r : running) {
            if (++gen[r] < output[r]) {
                kept.push_back(r);
                continue;
            }
            const int rc = mem.release(r);
            if (rc) return rc;
            finish[r] = t;
            ++finished;
        }
        running.swap(kept);
        int64_t admitted = 0, blocked = 0;
        while (!waiting.empty() && static_cast<int64_t>(running.size()) < max_batch) {
            const int32_t h = waiting.front();
            const int64_t tokens = static_cast<int64_t>(prompt[h]) + gen[h];
            bool ok = false;
            const int rc = mem.admit(h, tokens, &ok);
            if (rc) return rc;
            if (!ok) {
                blocked = mem.need(h, tokens);
                break;
            }
            waiting.pop_front();
            running.push_back(h);
            ++admitted;
        }
        int64_t used = 0, final_sum = 0;
        for (const int32_t r : running) {
            used += static_cast<int64_t>(prompt[r]) + gen[r];
            final_sum += static_cast<int64_t>(prompt[r]) + output[r];
        }
        const int64_t held = mem.held();
        int64_t *row = trace + t * kFields;
        row[kStep] = t;
        row[kRunning] = static_cast<int64_t>(running.size());
        row[kWaiting] = static_cast<int64_t>(waiting.size());
        row[kUsed] = used;
        row[kHeld] = held;
        row[kFree] = capacity - held;
        row[kLargestFree] = mem.largest_free();
        row[kAdmitted] = admitted;
        row[kPreempted] = preempted;
        row[kFinished] = finished;
        row[kDecoded] = decoded;
        row[kBlockedNeed] = blocked;
        row[kFinalSum] = final_sum;
        if (next == n && waiting.empty() && running.empty()) {
            *n_steps_out = t + 1;
            return PKV_OK;
        }
    }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_sim_paged(int32_t num_blocks, int32_t block_size, int32_t watermark_blocks, int32_t max_batch,
                             const int32_t *arrival, const int32_t *prompt_len, const int32_t *output_len,
                             int32_t n_requests, int64_t max_steps, int64_t *trace_out, int64_t *n_steps_out,
                             int64_t *finish_out) {
    const char *fn = "pkv_sim_paged";
    if (num_blocks <= 0 || block_size <= 0 || watermark_blocks < 0 || max_batch <= 0 || max_steps <= 0 ||
        !trace_out || !n_steps_out || (n_requests > 0 && !finish_out))
        return fail(PKV_EINVAL, "%s: bad arguments", fn);
    int rc = check_requests(fn, arrival, prompt_len, output_len, n_requests);
    if (rc) return rc;
    for (int32_t i = 0; i < n_requests; ++i)
        if (ceil_div(static_cast<int64_t>(prompt_len[i]) + output_len[i], block_size) + watermark_blocks > num_blocks)
            return fail(PKV_EINVAL, "%s: request %d (%d + %d tokens) can never fit %d blocks with %d kept free", fn, i,
                        prompt_len[i], output_len[i], num_blocks, watermark_blocks);
    pkv_pool *pool = nullptr;
    rc = pkv_pool_create(num_blocks, block_size, nullptr, &pool);
    if (rc) return rc;
    PagedMemory mem(pool, block_size, num_blocks, watermark_blocks);
    rc = run(fn, mem, static_cast<int64_t>(num_blocks) * block_size, max_batch, arrival, prompt_len, output_len,
             n_requests, max_steps, trace_out, n_steps_out, finish_out);
    pkv_pool_destroy(pool);
    return rc;
}

extern "C" int pkv_sim_contiguous(int64_t capacity, int32_t max_batch, const int32_t *arrival,
                                  const int32_t *prompt_len, const int32_t *output_len, const int32_t *reserve_len,
                                  int32_t n_requests, int64_t max_steps, int64_t *trace_out, int64_t *n_steps_out,
                                  int64_t *finish_out) {
    const char *fn = "pkv_sim_contiguous";
    if (capacity <= 0 || max_batch <= 0 || max_steps <= 0 || !trace_out || !n_steps_out ||
        (n_requests > 0 && (!finish_out || !reserve_len)))
        return fail(PKV_EINVAL, "%s: bad arguments", fn);
    int rc = check_requests(fn, arrival, prompt_len, output_len, n_requests);
    if (rc) return rc;
    for (int32_t i = 0; i < n_requests; ++i)
        if (reserve_len[i] < static_cast<int64_t>(prompt_len[i]) + output_len[i] || reserve_len[i] > capacity)
            return fail(PKV_EINVAL, "%s: reserve_len[%d] = %d must cover %d + %d tokens and fit %lld slots", fn, i,
                        reserve_len[i], prompt_len[i], output_len[i], static_cast<long long>(capacity));
    ContiguousMemory mem(capacity, reserve_len);
    return run(fn, mem, capacity, max_batch, arrival, prompt_len, output_len, n_requests, max_steps, trace_out,
               n_steps_out, finish_out);
}
