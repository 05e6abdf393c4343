// Host-side bookkeeping of a paged KV cache: block tables, reference counts, a
// free queue, prefix caching of full blocks, fork and copy-on-write.
//
// What it implements ("Forward Deployed Engineering Interview", Ch.2 section 8,
// the block-manager teaching model; "Anthropic Interview: Design an LLM
// Inference API with GPU Batching", 4.1/4.2 data model):
//   * a block holds 16 token slots, a reference count and the token ids
//     written to it; a full block also gets a prefix key;
//   * the key of a full block covers its parent's key (the block before it in
//     the table) and its own tokens; a first block starts from the sequence's
//     salt, so a different salt, or one changed early token, changes every key
//     after it; keyed blocks are found through the prefix cache;
//   * admitting a prompt reuses cached blocks for the unbroken run of full
//     blocks at its start (taking released ones back out of the free queue)
//     and takes fresh blocks for the rest;
//   * taking a block pops the front of the free queue (least recently freed)
//     and drops the cache entry the block still carried;
//   * appending opens a fresh block when the last one is full and copies the
//     last block first when it is shared: a shared block is never written;
//   * fork shares every block with the child; release drops one reference per
//     block, last block first, and a block left unreferenced joins the back of
//     the free queue, still cached until it is taken again.
// An operation that needs more free blocks than there are fails with
// KV_ERR_NO_BLOCKS and changes nothing.
//
// Prefix keys are SHA-256 digests (FIPS 180-4) of a fixed-layout encoding:
// 'S' salt | tokens for a first block, 'P' parent digest | tokens otherwise,
// tokens as 16 little-endian int32.
#include <algorithm>
#include <array>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "errors.h"
#include "pagedkv.h"

namespace pagedkv {
namespace {

constexpr int kBlock = 16;

// ---------------------------------------------------------------- SHA-256
class Sha256 {
 public:
  void update(const void* data, size_t n) {
    const uint8_t* p = static_cast<const uint8_t*>(data);
    len_ += n;
    while (n > 0) {
      const size_t take = std::min(n, size_t(64) - fill_);
      std::memcpy(buf_ + fill_, p, take);
      fill_ += take;
      p += take;
      n -= take;
      if (fill_ == 64) {
        compress(buf_);
        fill_ = 0;
      }
    }
  }
  std::array<uint8_t, 32> finish() {
    const uint64_t bits = uint64_t(len_) * 8;
    const uint8_t one = 0x80;
    update(&one, 1);
    const uint8_t zero = 0;
    while (fill_ != 56) update(&zero, 1);
    uint8_t be[8];
    for (int i = 0; i < 8; ++i) be[i] = uint8_t(bits >> (56 - 8 * i));
    update(be, 8);
    std::array<uint8_t, 32> out{};
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) out[4 * i + j] = uint8_t(h_[i] >> (24 - 8 * j));
    return out;
  }

 private:
  static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }
  void compress(const uint8_t* blk) {
    static const uint32_t k[64] = {
        0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4,
        0xab1c5ed5, 0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe,
        0x9bdc06a7, 0xc19bf174, 0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f,
        0x4a7484aa, 0x5cb0a9dc, 0x76f988da, 0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7,
        0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967, 0x27b70a85, 0x2e1b2138, 0x4d2c6dfc,
        0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85, 0xa2bfe8a1, 0xa81a664b,
        0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070, 0x19a4c116,
        0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
        0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7,
        0xc67178f2};
    uint32_t w[64];
    for (int i = 0; i < 16; ++i)
      w[i] = uint32_t(blk[4 * i]) << 24 | uint32_t(blk[4 * i + 1]) << 16 |
             uint32_t(blk[4 * i + 2]) << 8 | uint32_t(blk[4 * i + 3]);
    for (int i = 16; i < 64; ++i) {
      const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
      const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
      w[i] = w[i - 16] + s0 + w[i - 7] + s1;
    }
    uint32_t a = h_[0], b = h_[1], c = h_[2], d = h_[3], e = h_[4], f = h_[5], g = h_[6],
             h = h_[7];
    for (int i = 0; i < 64; ++i) {
      const uint32_t t1 = h + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & f) ^ (~e & g)) +
                          k[i] + w[i];
      const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) ^ (a & c) ^ (b & c));
      h = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h_[0] += a; h_[1] += b; h_[2] += c; h_[3] += d;
    h_[4] += e; h_[5] += f; h_[6] += g; h_[7] += h;
  }
  uint32_t h_[8] = {0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a,
                    0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19};
  uint8_t buf_[64];
  size_t fill_ = 0;
  size_t len_ = 0;
};

using Digest = std::array<uint8_t, 32>;
struct DigestHash {
  size_t operator()(const Digest& d) const {
    size_t h;
    std::memcpy(&h, d.data(), sizeof(h));
    return h;
  }
};

Digest prefix_key(const Digest* parent, const std::string& salt, const int32_t* tokens) {
  Sha256 s;
  if (parent) {
    s.update("P", 1);
    s.update(parent->data(), parent->size());
  } else {
    s.update("S", 1);
    s.update(salt.data(), salt.size());
  }
  s.update("|", 1);
  uint8_t le[4 * kBlock];
  for (int i = 0; i < kBlock; ++i)
    for (int j = 0; j < 4; ++j) le[4 * i + j] = uint8_t(uint32_t(tokens[i]) >> (8 * j));
  s.update(le, sizeof(le));
  return s.finish();
}

struct Block {
  int32_t refs = 0;
  int32_t ntok = 0;
  int32_t tokens[kBlock] = {};
  bool keyed = false;
  Digest key{};
  // free-queue links (-1 = none) and membership
  int32_t prev = -1, next = -1;
  bool in_free = false;
};

}  // namespace

class BlockManager {
 public:
  explicit BlockManager(int32_t n) : blocks_(size_t(n)) {
    for (int32_t i = 0; i < n; ++i) push_back_free(i);
  }

  int32_t num_free() const { return free_count_; }

  // Cached blocks the prompt would reuse and fresh blocks it would need.
  void plan_admit(const int32_t* tokens, int32_t n, const std::string& salt,
                  std::vector<int32_t>& reuse, int32_t& fresh) const {
    reuse.clear();
    const int32_t chunks = (n + kBlock - 1) / kBlock;
    const Digest* parent = nullptr;
    for (int32_t c = 0; c < chunks; ++c) {
      if (n - c * kBlock < kBlock) break;  // a partial chunk is never cached
      const Digest k = prefix_key(parent, salt, tokens + c * kBlock);
      auto it = cache_.find(k);
      if (it == cache_.end()) break;
      reuse.push_back(it->second);
      parent = &blocks_[size_t(it->second)].key;
    }
    fresh = chunks - int32_t(reuse.size());
  }

  kv_status admit(int64_t seq, const int32_t* tokens, int32_t n, std::string salt, int32_t* hits) {
    if (seqs_.count(seq)) return KV_ERR_INVALID_ARG;
    std::vector<int32_t> reuse;
    int32_t fresh = 0;
    plan_admit(tokens, n, salt, reuse, fresh);
    int32_t revived = 0;
    for (int32_t b : reuse) revived += blocks_[size_t(b)].refs == 0;
    if (fresh > free_count_ - revived) return KV_ERR_NO_BLOCKS;
    Seq s;
    s.salt = std::move(salt);
    for (int32_t b : reuse) {
      Block& blk = blocks_[size_t(b)];
      if (blk.refs == 0) unlink_free(b);
      ++blk.refs;
      s.table.push_back(b);
    }
    for (int32_t c = int32_t(reuse.size()); c < int32_t(reuse.size()) + fresh; ++c) {
      const int32_t cnt = std::min(kBlock, n - c * kBlock);
      const int32_t b = take(tokens + c * kBlock, cnt);
      seal(b, s.table.empty() ? -1 : s.table.back(), s.salt);
      s.table.push_back(b);
    }
    *hits = int32_t(reuse.size()) * kBlock;
    seqs_.emplace(seq, std::move(s));
    return KV_OK;
  }

  kv_status append(int64_t seq, int32_t token, int64_t* slot, int32_t* copy_src,
                   int32_t* copy_dst) {
    auto it = seqs_.find(seq);
    if (it == seqs_.end()) return KV_ERR_INVALID_ARG;
    Seq& s = it->second;
    *copy_src = -1;
    *copy_dst = -1;
    const int32_t last = s.table.empty() ? -1 : s.table.back();
    if (last < 0 || blocks_[size_t(last)].ntok == kBlock) {
      if (free_count_ == 0) return KV_ERR_NO_BLOCKS;
      s.table.push_back(take(nullptr, 0));
    } else if (blocks_[size_t(last)].refs > 1) {  // copy-on-write
      if (free_count_ == 0) return KV_ERR_NO_BLOCKS;
      Block& old = blocks_[size_t(last)];
      --old.refs;
      const int32_t nb = take(old.tokens, old.ntok);
      *copy_src = last;
      *copy_dst = nb;
      s.table.back() = nb;
    }
    const int32_t b = s.table.back();
    Block& blk = blocks_[size_t(b)];
    blk.tokens[blk.ntok++] = token;
    seal(b, s.table.size() > 1 ? s.table[s.table.size() - 2] : -1, s.salt);
    *slot = int64_t(b) * kBlock + blk.ntok - 1;
    return KV_OK;
  }

  kv_status fork(int64_t seq, int64_t child) {
    auto it = seqs_.find(seq);
    if (it == seqs_.end() || seqs_.count(child)) return KV_ERR_INVALID_ARG;
    for (int32_t b : it->second.table) ++blocks_[size_t(b)].refs;
    Seq copy = it->second;
    seqs_.emplace(child, std::move(copy));
    return KV_OK;
  }

  kv_status release(int64_t seq) {
    auto it = seqs_.find(seq);
    if (it == seqs_.end()) return KV_ERR_INVALID_ARG;
    const std::vector<int32_t>& t = it->second.table;
    for (auto b = t.rbegin(); b != t.rend(); ++b)
      if (--blocks_[size_t(*b)].refs == 0) push_back_free(*b);
    seqs_.erase(it);
    return KV_OK;
  }

  kv_status table(int64_t seq, int32_t* out, int32_t cap, int32_t* nblocks,
                  int32_t* ntokens) const {
    auto it = seqs_.find(seq);
    if (it == seqs_.end()) return KV_ERR_INVALID_ARG;
    const std::vector<int32_t>& t = it->second.table;
    if (nblocks) *nblocks = int32_t(t.size());
    if (ntokens)
      *ntokens = t.empty() ? 0 : int32_t(t.size() - 1) * kBlock + blocks_[size_t(t.back())].ntok;
    if (out) {
      if (cap < int32_t(t.size())) return KV_ERR_INVALID_ARG;
      for (size_t i = 0; i < t.size(); ++i) out[i] = t[i];
    }
    return KV_OK;
  }

  std::mutex mu;

 private:
  struct Seq {
    std::vector<int32_t> table;
    std::string salt;
  };

  int32_t take(const int32_t* tokens, int32_t n) {
    const int32_t b = free_head_;
    unlink_free(b);
    Block& blk = blocks_[size_t(b)];
    if (blk.keyed) {
      auto it = cache_.find(blk.key);
      if (it != cache_.end() && it->second == b) cache_.erase(it);
    }
    blk.refs = 1;
    blk.ntok = n;
    for (int32_t i = 0; i < n; ++i) blk.tokens[i] = tokens[i];
    blk.keyed = false;
    return b;
  }

  void seal(int32_t b, int32_t parent, const std::string& salt) {
    Block& blk = blocks_[size_t(b)];
    if (blk.ntok != kBlock) return;
    blk.key = prefix_key(parent >= 0 ? &blocks_[size_t(parent)].key : nullptr, salt, blk.tokens);
    blk.keyed = true;
    cache_.emplace(blk.key, b);  // an existing entry is kept
  }

  void push_back_free(int32_t b) {
    Block& blk = blocks_[size_t(b)];
    blk.prev = free_tail_;
    blk.next = -1;
    if (free_tail_ >= 0) blocks_[size_t(free_tail_)].next = b; else free_head_ = b;
    free_tail_ = b;
    blk.in_free = true;
    ++free_count_;
  }

  void unlink_free(int32_t b) {
    Block& blk = blocks_[size_t(b)];
    if (blk.prev >= 0) blocks_[size_t(blk.prev)].next = blk.next; else free_head_ = blk.next;
    if (blk.next >= 0) blocks_[size_t(blk.next)].prev = blk.prev; else free_tail_ = blk.prev;
    blk.prev = blk.next = -1;
    blk.in_free = false;
    --free_count_;
  }

  std::vector<Block> blocks_;
  int32_t free_head_ = -1, free_tail_ = -1, free_count_ = 0;
  std::unordered_map<Digest, int32_t, DigestHash> cache_;
  std::unordered_map<int64_t, Seq> seqs_;
};

}  // namespace pagedkv

struct kv_block_manager {
  pagedkv::BlockManager impl;
  explicit kv_block_manager(int32_t n) : impl(n) {}
};

namespace {
constexpr int32_t kMaxBlocks = 1 << 28;

kv_status check(kv_status s, const char* what, int64_t seq) {
  if (s == KV_OK) return pagedkv::report_ok();
  if (s == KV_ERR_NO_BLOCKS)
    return pagedkv::report(s, "%s of sequence %lld: not enough free blocks", what,
                           static_cast<long long>(seq));
  return pagedkv::report(s, "%s: bad sequence id %lld", what, static_cast<long long>(seq));
}
}  // namespace

extern "C" {

kv_status kv_bm_create(int32_t num_blocks, kv_block_manager** out) {
  using pagedkv::report;
  if (!out) return report(KV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || num_blocks > kMaxBlocks)
    return report(KV_ERR_INVALID_ARG, "num_blocks %d outside [1, %d]", num_blocks, kMaxBlocks);
  *out = new (std::nothrow) kv_block_manager(num_blocks);
  return *out ? pagedkv::report_ok() : report(KV_ERR_INVALID_ARG, "out of host memory");
}

void kv_bm_destroy(kv_block_manager* bm) { delete bm; }

kv_status kv_bm_admit(kv_block_manager* bm, int64_t seq, const int32_t* tokens, int32_t n,
                      const char* salt, int32_t salt_len, int32_t* hits) {
  if (!bm || !hits || n < 0 || (n > 0 && !tokens) || salt_len < 0 || (salt_len > 0 && !salt))
    return pagedkv::report(KV_ERR_INVALID_ARG, "admit: bad argument (manager, hits, tokens, n, salt)");
  std::lock_guard<std::mutex> lock(bm->impl.mu);
  return check(bm->impl.admit(seq, tokens, n, std::string(salt ? salt : "", size_t(salt_len)), hits),
               "admit", seq);
}

kv_status kv_bm_append(kv_block_manager* bm, int64_t seq, int32_t token, int64_t* slot,
                       int32_t* copy_src, int32_t* copy_dst) {
  if (!bm || !slot || !copy_src || !copy_dst)
    return pagedkv::report(KV_ERR_INVALID_ARG, "append: NULL argument");
  std::lock_guard<std::mutex> lock(bm->impl.mu);
  return check(bm->impl.append(seq, token, slot, copy_src, copy_dst), "append", seq);
}

kv_status kv_bm_append_batch(kv_block_manager* bm, const int64_t* seqs, const int32_t* tokens,
                             int32_t B, int64_t* slots, int32_t* copy_src, int32_t* copy_dst,
                             int32_t* n_copies, int32_t* done) {
  if (done) *done = 0;
  if (!bm || B < 0 || !n_copies || (B > 0 && (!seqs || !tokens || !slots || !copy_src || !copy_dst)))
    return pagedkv::report(KV_ERR_INVALID_ARG, "append_batch: bad argument");
  std::lock_guard<std::mutex> lock(bm->impl.mu);
  *n_copies = 0;
  for (int32_t b = 0; b < B; ++b) {
    int32_t cs = -1, cd = -1;
    const kv_status s = bm->impl.append(seqs[b], tokens[b], &slots[b], &cs, &cd);
    if (s != KV_OK) return check(s, "append_batch", seqs[b]);
    if (cs >= 0) {
      copy_src[*n_copies] = cs;
      copy_dst[*n_copies] = cd;
      ++*n_copies;
    }
    if (done) *done = b + 1;
  }
  return pagedkv::report_ok();
}

kv_status kv_bm_fork(kv_block_manager* bm, int64_t seq, int64_t child) {
  if (!bm) return pagedkv::report(KV_ERR_INVALID_ARG, "fork: manager is NULL");
  std::lock_guard<std::mutex> lock(bm->impl.mu);
  return check(bm->impl.fork(seq, child), "fork (unknown parent or existing child)", seq);
}

kv_status kv_bm_release(kv_block_manager* bm, int64_t seq) {
  if (!bm) return pagedkv::report(KV_ERR_INVALID_ARG, "release: manager is NULL");
  std::lock_guard<std::mutex> lock(bm->impl.mu);
  return check(bm->impl.release(seq), "release", seq);
}

int32_t kv_bm_num_free(kv_block_manager* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->impl.mu);
  return bm->impl.num_free();
}

kv_status kv_bm_table(kv_block_manager* bm, int64_t seq, int32_t* blocks, int32_t capacity,
                      int32_t* num_blocks, int32_t* num_tokens) {
  if (!bm || capacity < 0) return pagedkv::report(KV_ERR_INVALID_ARG, "table: bad argument");
  std::lock_guard<std::mutex> lock(bm->impl.mu);
  return check(bm->impl.table(seq, blocks, capacity, num_blocks, num_tokens),
               "table (unknown sequence or capacity too small)", seq);
}

kv_status kv_bm_batch_tables(kv_block_manager* bm, const int64_t* seqs, int32_t B, int32_t max_nb,
                             int32_t* tables, int32_t* context_lens) {
  if (!bm || B < 0 || max_nb < 1 || (B > 0 && (!seqs || !tables || !context_lens)))
    return pagedkv::report(KV_ERR_INVALID_ARG, "batch_tables: bad argument");
  std::lock_guard<std::mutex> lock(bm->impl.mu);
  for (int32_t b = 0; b < B; ++b) {
    int32_t nb = 0, nt = 0;
    if (bm->impl.table(seqs[b], nullptr, 0, &nb, &nt) != KV_OK)
      return pagedkv::report(KV_ERR_INVALID_ARG, "batch_tables: unknown sequence %lld",
                             static_cast<long long>(seqs[b]));
    if (nb > max_nb)
      return pagedkv::report(KV_ERR_INVALID_ARG, "batch_tables: sequence %lld has %d blocks > %d",
                             static_cast<long long>(seqs[b]), nb, max_nb);
  }
  for (int32_t b = 0; b < B; ++b) {
    int32_t* row = tables + int64_t(b) * max_nb;
    int32_t nb = 0;
    bm->impl.table(seqs[b], row, max_nb, &nb, &context_lens[b]);
    for (int32_t j = nb; j < max_nb; ++j) row[j] = -1;
  }
  return pagedkv::report_ok();
}

}  // extern "C"
