// Test driver of libpa's host code (the block allocator, the host validators and planners, the error
// strings), built on its own with g++ -fsanitize=address,undefined so that every call the
// differential tests make runs under the sanitizers.  Only tests/ builds and runs it.
//
// Protocol: one request per line on stdin, whitespace-separated integers after a command word;
// an array is sent as its length followed by its elements.  Each reply is one line: "0 <outputs>"
// on success, or "<status> <message>" on failure.  Every output buffer is a heap allocation of
// exactly the capacity the call is given, so a write past it is caught by the address sanitizer.
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <map>
#include <memory>
#include <sstream>
#include <stdexcept>
#include <string>

#include "pa.h"

namespace {

std::map<int64_t, pa_allocator*> handles;
int64_t next_handle = 1;

// An array of exactly n elements in its own heap allocation (new T[0] included), so any access past
// the end, even of an empty array, is reported by the address sanitizer.
template <class T>
struct Buf {
  std::unique_ptr<T[]> p;
  int64_t n = 0;
  T* data() const { return p.get(); }
  int64_t size() const { return n; }
  bool empty() const { return n == 0; }
  T& operator[](int64_t k) const { return p[k]; }
};

template <class T>
Buf<T> buf(int64_t n) {
  n = n > 0 ? n : 0;
  return Buf<T>{std::unique_ptr<T[]>(new T[static_cast<size_t>(n)]()), n};
}

struct Line {
  std::istringstream in;
  explicit Line(const std::string& s) : in(s) {}
  int64_t i() {
    int64_t v = 0;
    if (!(in >> v)) throw std::runtime_error("short request");
    return v;
  }
  template <class T>
  Buf<T> arr() {
    const int64_t n = i();
    if (n < 0) throw std::runtime_error("negative array length");
    Buf<T> v = buf<T>(n);
    for (int64_t k = 0; k < n; ++k) v[k] = static_cast<T>(i());
    return v;
  }
};

pa_allocator* H(Line& l) {
  auto it = handles.find(l.i());
  if (it == handles.end()) throw std::runtime_error("unknown handle");
  return it->second;
}

template <class T>
void put(std::ostringstream& o, const Buf<T>& v, int64_t n) {
  o << ' ' << n;
  for (int64_t k = 0; k < n; ++k) o << ' ' << static_cast<int64_t>(v[k]);
}

std::string reply(pa_status st, const std::ostringstream& o) {
  if (st != PA_OK) return std::to_string(st) + " " + pa_last_error();
  return "0" + o.str();
}

std::string run(const std::string& cmd, Line& l) {
  std::ostringstream o;
  if (cmd == "create") {
    const int32_t nb = static_cast<int32_t>(l.i()), bs = static_cast<int32_t>(l.i());
    auto order = l.arr<int32_t>();
    pa_allocator* a = nullptr;
    const pa_status st = pa_alloc_create(nb, bs, order.empty() ? nullptr : order.data(), &a);
    if (st == PA_OK) {
      handles[next_handle] = a;
      o << ' ' << next_handle++;
    }
    return reply(st, o);
  }
  if (cmd == "destroy") {
    const int64_t h = l.i();
    auto it = handles.find(h);
    if (it != handles.end()) {
      pa_alloc_destroy(it->second);
      handles.erase(it);
    }
    return "0";
  }
  if (cmd == "add") {
    pa_allocator* a = H(l);
    return reply(pa_alloc_add_seq(a, l.i()), o);
  }
  if (cmd == "fork") {
    pa_allocator* a = H(l);
    const int64_t p = l.i(), c = l.i();
    return reply(pa_alloc_fork(a, p, c), o);
  }
  if (cmd == "free") {
    pa_allocator* a = H(l);
    return reply(pa_alloc_free_seq(a, l.i()), o);
  }
  if (cmd == "append") {            // append h sid n cow_cap
    pa_allocator* a = H(l);
    const int64_t sid = l.i();
    const int32_t n = static_cast<int32_t>(l.i()), cap = static_cast<int32_t>(l.i());
    auto slots = buf<int64_t>(n);
    auto cow = buf<int32_t>(2 * static_cast<int64_t>(cap));
    int32_t ncow = 0;
    const pa_status st = pa_alloc_append(a, sid, n, slots.data(), cow.data(), cap, &ncow);
    put(o, slots, n);
    put(o, cow, 2 * static_cast<int64_t>(ncow));
    return reply(st, o);
  }
  if (cmd == "batch") {             // batch h [sids] [ns] cow_cap
    pa_allocator* a = H(l);
    auto sids = l.arr<int64_t>();
    auto ns = l.arr<int32_t>();
    const int32_t cap = static_cast<int32_t>(l.i());
    if (sids.size() != ns.size()) throw std::runtime_error("batch arrays disagree");
    int64_t total = 0;
    for (int64_t k = 0; k < ns.size(); ++k) total += ns[k] > 0 ? ns[k] : 0;
    auto slots = buf<int64_t>(total);
    auto cow = buf<int32_t>(2 * static_cast<int64_t>(cap));
    int32_t ncow = 0;
    const pa_status st = pa_alloc_append_batch(a, sids.data(), ns.data(), static_cast<int32_t>(sids.size()),
                                               slots.data(), cow.data(), cap, &ncow);
    put(o, slots, total);
    put(o, cow, 2 * static_cast<int64_t>(ncow));
    return reply(st, o);
  }
  if (cmd == "needed") {
    pa_allocator* a = H(l);
    const int64_t sid = l.i();
    int32_t out = 0;
    const pa_status st = pa_alloc_blocks_needed(a, sid, static_cast<int32_t>(l.i()), &out);
    o << ' ' << out;
    return reply(st, o);
  }
  if (cmd == "len") {
    pa_allocator* a = H(l);
    int64_t out = 0;
    const pa_status st = pa_alloc_seq_len(a, l.i(), &out);
    o << ' ' << out;
    return reply(st, o);
  }
  if (cmd == "table") {             // table h sid cap
    pa_allocator* a = H(l);
    const int64_t sid = l.i();
    const int32_t cap = static_cast<int32_t>(l.i());
    auto out = buf<int32_t>(cap);
    int32_t n = 0;
    const pa_status st = pa_alloc_block_table(a, sid, out.data(), cap, &n);
    put(o, out, st == PA_OK ? n : 0);
    return reply(st, o);
  }
  if (cmd == "fill") {              // fill h [sids] max_blocks pad
    pa_allocator* a = H(l);
    auto sids = l.arr<int64_t>();
    const int32_t mb = static_cast<int32_t>(l.i()), pad = static_cast<int32_t>(l.i());
    const int64_t n = static_cast<int64_t>(sids.size()) * mb;
    auto out = buf<int32_t>(n);
    const pa_status st = pa_alloc_fill_tables(a, sids.data(), static_cast<int32_t>(sids.size()), out.data(), mb, pad);
    put(o, out, st == PA_OK ? n : 0);
    return reply(st, o);
  }
  if (cmd == "ref") {
    pa_allocator* a = H(l);
    int32_t out = 0;
    const pa_status st = pa_alloc_refcount(a, static_cast<int32_t>(l.i()), &out);
    o << ' ' << out;
    return reply(st, o);
  }
  if (cmd == "stats") {
    pa_allocator* a = H(l);
    int32_t f = 0, u = 0;
    int64_t r = 0;
    const pa_status st = pa_alloc_stats(a, &f, &u, &r);
    o << ' ' << f << ' ' << u << ' ' << r;
    return reply(st, o);
  }
  if (cmd == "freelist" || cmd == "evictable") {   // freelist h cap
    pa_allocator* a = H(l);
    const int32_t cap = static_cast<int32_t>(l.i());
    auto out = buf<int32_t>(cap);
    int32_t n = 0;
    const pa_status st = cmd == "freelist" ? pa_alloc_free_list(a, out.data(), cap, &n)
                                           : pa_alloc_evictable_list(a, out.data(), cap, &n);
    put(o, out, st == PA_OK ? n : 0);
    return reply(st, o);
  }
  if (cmd == "prefix_on") return reply(pa_alloc_enable_prefix_cache(H(l)), o);
  if (cmd == "addprefix") {         // addprefix h sid [tokens]
    pa_allocator* a = H(l);
    const int64_t sid = l.i();
    auto tok = l.arr<int32_t>();
    int32_t n = 0;
    const pa_status st = pa_alloc_add_seq_prefix(a, sid, tok.data(), static_cast<int32_t>(tok.size()), &n);
    o << ' ' << n;
    return reply(st, o);
  }
  if (cmd == "cache") {             // cache h sid [tokens]
    pa_allocator* a = H(l);
    const int64_t sid = l.i();
    auto tok = l.arr<int32_t>();
    return reply(pa_alloc_cache_seq(a, sid, tok.data(), tok.size()), o);
  }
  if (cmd == "cstats") {
    pa_allocator* a = H(l);
    int32_t c = 0, e = 0;
    const pa_status st = pa_alloc_cache_stats(a, &c, &e);
    o << ' ' << c << ' ' << e;
    return reply(st, o);
  }
  if (cmd == "move") {              // move src dst sid cap
    pa_allocator* s = H(l);
    pa_allocator* d = H(l);
    const int64_t sid = l.i();
    const int32_t cap = static_cast<int32_t>(l.i());
    auto out = buf<int32_t>(2 * static_cast<int64_t>(cap));
    int32_t n = 0;
    const pa_status st = pa_alloc_move_seq(s, d, sid, out.data(), cap, &n);
    put(o, out, st == PA_OK ? 2 * static_cast<int64_t>(n) : 0);
    return reply(st, o);
  }
  // host validators: the pool is sent as num_blocks block_size
  if (cmd == "vdecode") {           // vdecode nb bs max_blocks [tables] [lens] max_context_len
    pa_pool_desc p{static_cast<int32_t>(l.i()), static_cast<int32_t>(l.i()), 1, 64, PA_BF16, 1.f, 1.f};
    const int32_t mb = static_cast<int32_t>(l.i());
    auto t = l.arr<int32_t>();
    auto lens = l.arr<int32_t>();
    const int32_t mx = static_cast<int32_t>(l.i());
    if (t.size() != lens.size() * mb)
      throw std::runtime_error("table size");
    return reply(pa_validate_decode(&p, t.data(), mb, lens.data(),
                                    static_cast<int32_t>(lens.size()), mx),
                 o);
  }
  if (cmd == "vprefill") {          // vprefill nb bs max_blocks [tables] [qsl] [prior] max_chunk total_q
    pa_pool_desc p{static_cast<int32_t>(l.i()), static_cast<int32_t>(l.i()), 1, 64, PA_BF16, 1.f, 1.f};
    const int32_t mb = static_cast<int32_t>(l.i());
    auto t = l.arr<int32_t>();
    auto qsl = l.arr<int32_t>();
    auto prior = l.arr<int32_t>();
    const int32_t mc = static_cast<int32_t>(l.i());
    const int64_t tq = l.i();
    if (qsl.size() != prior.size() + 1 || t.size() != prior.size() * mb)
      throw std::runtime_error("prefill sizes");
    return reply(pa_validate_prefill(&p, t.data(), mb, qsl.data(),
                                     prior.data(), static_cast<int32_t>(prior.size()), mc,
                                     tq),
                 o);
  }
  if (cmd == "vslots") {            // vslots nb bs [slots]
    pa_pool_desc p{static_cast<int32_t>(l.i()), static_cast<int32_t>(l.i()), 1, 64, PA_BF16, 1.f, 1.f};
    auto s = l.arr<int64_t>();
    return reply(pa_validate_slots(&p, s.data(), s.size()), o);
  }
  if (cmd == "vpairs") {            // vpairs nb_src nb_dst [pairs] in_place
    pa_pool_desc ps{static_cast<int32_t>(l.i()), 16, 1, 64, PA_BF16, 1.f, 1.f};
    pa_pool_desc pd{static_cast<int32_t>(l.i()), 16, 1, 64, PA_BF16, 1.f, 1.f};
    auto pr = l.arr<int32_t>();
    const int32_t in_place = static_cast<int32_t>(l.i());
    return reply(pa_validate_pairs(&ps, &pd, pr.data(), static_cast<int32_t>(pr.size() / 2),
                                   in_place),
                 o);
  }
  if (cmd == "hint") {              // hint max_blocks [tables] [lens] block_size
    const int32_t mb = static_cast<int32_t>(l.i());
    auto t = l.arr<int32_t>();
    auto lens = l.arr<int32_t>();
    const int32_t bs = static_cast<int32_t>(l.i());
    if (t.size() != lens.size() * mb) throw std::runtime_error("table size");
    auto out = buf<int32_t>(lens.size());
    const pa_status st = pa_plan_cache_hint(t.data(), mb, lens.data(), static_cast<int32_t>(lens.size()), bs, out.data());
    put(o, out, st == PA_OK ? lens.size() : 0);
    return reply(st, o);
  }
  if (cmd == "tails") {             // tails max_blocks [tables] [lens] block_size width [shared]
    const int32_t mb = static_cast<int32_t>(l.i());
    auto t = l.arr<int32_t>();
    auto lens = l.arr<int32_t>();
    const int32_t bs = static_cast<int32_t>(l.i()), w = static_cast<int32_t>(l.i());
    auto shared = l.arr<int32_t>();
    const int32_t n = static_cast<int32_t>(lens.size());
    if (t.size() != static_cast<int64_t>(n) * mb) throw std::runtime_error("table size");
    auto ks = buf<int32_t>(w > 0 ? n / w : 0);
    pa_status st = pa_plan_shared_blocks(t.data(), mb, lens.data(), n, bs, w, ks.data());
    if (st != PA_OK) return reply(st, o);
    if (!shared.empty()) ks = std::move(shared);   // a caller's own (possibly wrong) counts
    auto tl = buf<int32_t>(n);
    int32_t need = 0;
    st = pa_plan_beam_tails(t.data(), mb, lens.data(), n, bs, w, ks.data(), nullptr, 0, tl.data(), &need);
    if (st != PA_OK) return reply(st, o);
    const int32_t cap = need > 0 ? need : 1;
    auto tt = buf<int32_t>(static_cast<int64_t>(n) * cap);
    st = pa_plan_beam_tails(t.data(), mb, lens.data(), n, bs, w, ks.data(), tt.data(), cap, tl.data(), nullptr);
    put(o, ks, w > 0 ? n / w : 0);
    o << ' ' << cap;
    put(o, tt, static_cast<int64_t>(n) * cap);
    put(o, tl, n);
    return reply(st, o);
  }
  throw std::runtime_error("unknown command " + cmd);
}

}  // namespace

int main() {
  std::ios::sync_with_stdio(false);
  std::string line;
  while (std::getline(std::cin, line)) {
    Line l(line);
    std::string cmd;
    if (!(l.in >> cmd)) continue;
    if (cmd == "quit") break;
    std::string out;
    try {
      out = run(cmd, l);
    } catch (const std::exception& e) {
      out = std::string("-1 driver: ") + e.what();
    }
    std::cout << out << '\n' << std::flush;
  }
  for (auto& kv : handles) pa_alloc_destroy(kv.second);
  return 0;
}
