// load_shard.hip -- tp_load_shard: one rank's shard of a tensor, read from a
// safetensors file straight into device memory.
//
// Diffusers "Tensor parallelism" page, "Load a sharded model": with a
// parallel config the checkpoint is sharded while it is read; every rank
// reads only its own slice of each weight and puts it on its GPU, so no rank
// ever holds a full-size weight.  "Limitations": this load takes safetensors
// weights only.
//
// safetensors layout (the format's published specification): an 8-byte
// little-endian header length H, then H bytes of JSON that map each tensor
// name to {"dtype", "shape", "data_offsets": [begin, end]} (byte offsets into
// the buffer that follows the header; an optional "__metadata__" entry maps
// strings to strings), then that byte buffer.  Tensors are row-major.
//
// Host code only.  The rank's slice is a sequence of byte runs of the file,
// each mapped to a contiguous range of the shard (one run per packed block for
// a colwise cut, one per row and block for a rowwise cut).  The runs are
// generated in shard order as the staging chunks are filled, never stored all
// at once, so the host memory of a load does not grow with the tensor's
// height.  A chunk is read with pread into one of two pinned staging buffers
// while the host-to-device copy of the other buffer runs on the caller's stream.
#include <errno.h>
#include <fcntl.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <exception>
#include <new>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include "tp_internal.h"
#include "tp_linear.h"

namespace {

// --------------------------------------------------------------------------
// A small strict JSON reader (RFC 8259 values), enough for the header.
// --------------------------------------------------------------------------
struct Json {
    enum Kind { Null, Bool, Number, String, Array, Object } kind = Null;
    bool b = false;
    bool is_int = false;  // an integer literal that fits int64
    int64_t i = 0;
    std::string s;
    std::vector<Json> a;
    std::vector<std::pair<std::string, Json>> o;

    const Json *get(const char *key) const
    {
        for (const auto &kv : o)
            if (kv.first == key)
                return &kv.second;
        return nullptr;
    }
};

class JsonReader {
  public:
    JsonReader(const char *p, const char *e) : p_(p), e_(e) {}

    bool parse(Json &out)
    {
        ws();
        if (!value(out, 0))
            return false;
        ws();
        return p_ == e_;
    }

  private:
    static constexpr int kMaxDepth = 32;
    // A safetensors header holds a few values per tensor; a cap on the values parsed
    // bounds the tree a malformed header can make the loader build in host memory.
    static constexpr int64_t kMaxValues = (int64_t)1 << 20;
    const char *p_, *e_;
    int64_t values_ = 0;

    void ws()
    {
        while (p_ < e_ && (*p_ == ' ' || *p_ == '\t' || *p_ == '\n' || *p_ == '\r'))
            ++p_;
    }
    bool literal(const char *lit)
    {
        const size_t n = strlen(lit);
        if ((size_t)(e_ - p_) < n || memcmp(p_, lit, n) != 0)
            return false;
        p_ += n;
        return true;
    }
    bool value(Json &v, int depth)
    {
        if (depth > kMaxDepth || p_ >= e_ || ++values_ > kMaxValues)
            return false;
        switch (*p_) {
        case '{': return object(v, depth);
        case '[': return array(v, depth);
        case '"': v.kind = Json::String; return string(v.s);
        case 't': v.kind = Json::Bool; v.b = true; return literal("true");
        case 'f': v.kind = Json::Bool; v.b = false; return literal("false");
        case 'n': v.kind = Json::Null; return literal("null");
        default: return number(v);
        }
    }
    bool object(Json &v, int depth)
    {
        v.kind = Json::Object;
        ++p_;
        ws();
        if (p_ < e_ && *p_ == '}') {
            ++p_;
            return true;
        }
        for (;;) {
            ws();
            std::string key;
            if (p_ >= e_ || *p_ != '"' || !string(key))
                return false;
            ws();
            if (p_ >= e_ || *p_ != ':')
                return false;
            ++p_;
            ws();
            Json child;
            if (!value(child, depth + 1))
                return false;
            v.o.emplace_back(std::move(key), std::move(child));
            ws();
            if (p_ >= e_)
                return false;
            if (*p_ == ',') {
                ++p_;
                continue;
            }
            if (*p_ == '}') {
                ++p_;
                return true;
            }
            return false;
        }
    }
    bool array(Json &v, int depth)
    {
        v.kind = Json::Array;
        ++p_;
        ws();
        if (p_ < e_ && *p_ == ']') {
            ++p_;
            return true;
        }
        for (;;) {
            ws();
            Json child;
            if (!value(child, depth + 1))
                return false;
            v.a.push_back(std::move(child));
            ws();
            if (p_ >= e_)
                return false;
            if (*p_ == ',') {
                ++p_;
                continue;
            }
            if (*p_ == ']') {
                ++p_;
                return true;
            }
            return false;
        }
    }
    static int hex(char c)
    {
        if (c >= '0' && c <= '9')
            return c - '0';
        if (c >= 'a' && c <= 'f')
            return c - 'a' + 10;
        if (c >= 'A' && c <= 'F')
            return c - 'A' + 10;
        return -1;
    }
    static void utf8(std::string &s, uint32_t cp)
    {
        if (cp < 0x80) {
            s.push_back((char)cp);
        } else if (cp < 0x800) {
            s.push_back((char)(0xC0 | (cp >> 6)));
            s.push_back((char)(0x80 | (cp & 0x3F)));
        } else if (cp < 0x10000) {
            s.push_back((char)(0xE0 | (cp >> 12)));
            s.push_back((char)(0x80 | ((cp >> 6) & 0x3F)));
            s.push_back((char)(0x80 | (cp & 0x3F)));
        } else {
            s.push_back((char)(0xF0 | (cp >> 18)));
            s.push_back((char)(0x80 | ((cp >> 12) & 0x3F)));
            s.push_back((char)(0x80 | ((cp >> 6) & 0x3F)));
            s.push_back((char)(0x80 | (cp & 0x3F)));
        }
    }
    bool hex4(uint32_t &cp)
    {
        if (e_ - p_ < 4)
            return false;
        cp = 0;
        for (int k = 0; k < 4; ++k) {
            const int h = hex(p_[k]);
            if (h < 0)
                return false;
            cp = cp * 16 + (uint32_t)h;
        }
        p_ += 4;
        return true;
    }
    bool string(std::string &s)
    {
        ++p_;  // the opening quote
        while (p_ < e_) {
            const char c = *p_++;
            if (c == '"')
                return true;
            if ((unsigned char)c < 0x20)
                return false;
            if (c != '\\') {
                s.push_back(c);
                continue;
            }
            if (p_ >= e_)
                return false;
            const char esc = *p_++;
            switch (esc) {
            case '"': case '\\': case '/': s.push_back(esc); break;
            case 'b': s.push_back('\b'); break;
            case 'f': s.push_back('\f'); break;
            case 'n': s.push_back('\n'); break;
            case 'r': s.push_back('\r'); break;
            case 't': s.push_back('\t'); break;
            case 'u': {
                uint32_t cp;
                if (!hex4(cp))
                    return false;
                if (cp >= 0xD800 && cp < 0xDC00) {  // high surrogate: a low one must follow
                    uint32_t lo;
                    if (e_ - p_ < 2 || p_[0] != '\\' || p_[1] != 'u')
                        return false;
                    p_ += 2;
                    if (!hex4(lo) || lo < 0xDC00 || lo >= 0xE000)
                        return false;
                    cp = 0x10000 + ((cp - 0xD800) << 10) + (lo - 0xDC00);
                } else if (cp >= 0xDC00 && cp < 0xE000) {
                    return false;
                }
                utf8(s, cp);
                break;
            }
            default: return false;
            }
        }
        return false;
    }
    static bool digit(char c) { return c >= '0' && c <= '9'; }
    bool number(Json &v)
    {
        v.kind = Json::Number;
        bool neg = false;
        if (p_ < e_ && *p_ == '-') {
            neg = true;
            ++p_;
        }
        if (p_ >= e_ || !digit(*p_))
            return false;
        uint64_t acc = 0;
        bool fits = true;
        if (*p_ == '0') {
            ++p_;
        } else {
            while (p_ < e_ && digit(*p_)) {
                const uint64_t d = (uint64_t)(*p_++ - '0');
                if (acc > (UINT64_C(0x7FFFFFFFFFFFFFFF) - d) / 10)
                    fits = false;
                else
                    acc = acc * 10 + d;
            }
        }
        bool integral = true;
        if (p_ < e_ && *p_ == '.') {
            integral = false;
            ++p_;
            if (p_ >= e_ || !digit(*p_))
                return false;
            while (p_ < e_ && digit(*p_))
                ++p_;
        }
        if (p_ < e_ && (*p_ == 'e' || *p_ == 'E')) {
            integral = false;
            ++p_;
            if (p_ < e_ && (*p_ == '+' || *p_ == '-'))
                ++p_;
            if (p_ >= e_ || !digit(*p_))
                return false;
            while (p_ < e_ && digit(*p_))
                ++p_;
        }
        v.is_int = integral && fits;
        v.i = neg ? -(int64_t)acc : (int64_t)acc;
        return true;
    }
};

// --------------------------------------------------------------------------
// Errors (the message buffer is the one tp_last_error() returns).
// --------------------------------------------------------------------------
__attribute__((format(printf, 2, 3))) tp_status fail(tp_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(tpl::last_error_buffer(), tpl::kLastErrorBytes, fmt, ap);
    va_end(ap);
    return s;
}

constexpr int64_t kMaxHeaderBytes = (int64_t)100 << 20;  // the header is JSON text: 100 MiB is ample
constexpr int64_t kStageBytes = (int64_t)32 << 20;       // each of the two pinned staging buffers
constexpr int kReadThreads = 8;                          // reader threads per staging chunk
constexpr int64_t kMinBytesPerThread = (int64_t)1 << 20; // below this a chunk is read by fewer threads
constexpr size_t kMaxChunkPieces = (size_t)1 << 16;      // pieces per staging chunk (tiny rowwise pieces)
constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int kMaxBlocks = 16;

bool read_full(int fd, void *buf, int64_t len, int64_t off)
{
    char *p = static_cast<char *>(buf);
    while (len > 0) {
        const size_t want = (size_t)(len < ((int64_t)1 << 30) ? len : ((int64_t)1 << 30));
        const ssize_t n = pread(fd, p, want, (off_t)off);
        if (n < 0) {
            if (errno == EINTR)
                continue;
            return false;
        }
        if (n == 0)
            return false;  // the file ended early
        p += n;
        off += n;
        len -= n;
    }
    return true;
}

struct TensorInfo {
    tp_dtype dtype;
    int es;
    int ndim;
    int64_t shape[2];
    int64_t data_begin;  // absolute file offset of the tensor's first byte
};

// Reads and checks the header; fills `ti` for tensor `name`.
tp_status read_tensor_info(const char *fn, const char *path, int fd, int64_t file_size, const char *name,
                           TensorInfo &ti)
{
    unsigned char len8[8];
    if (file_size < 8 || !read_full(fd, len8, 8, 0))
        return fail(TP_ERR_IO, "%s: %s: too short for a safetensors header", fn, path);
    uint64_t hlen = 0;
    for (int k = 7; k >= 0; --k)
        hlen = (hlen << 8) | len8[k];
    if (hlen == 0 || hlen > (uint64_t)kMaxHeaderBytes || (int64_t)hlen > file_size - 8)
        return fail(TP_ERR_IO, "%s: %s: header length %llu is outside the file or above %lld bytes", fn, path,
                    (unsigned long long)hlen, (long long)kMaxHeaderBytes);
    std::string text((size_t)hlen, '\0');
    if (!read_full(fd, &text[0], (int64_t)hlen, 8))
        return fail(TP_ERR_IO, "%s: %s: cannot read the header", fn, path);
    Json root;
    JsonReader reader(text.data(), text.data() + text.size());
    if (!reader.parse(root) || root.kind != Json::Object)
        return fail(TP_ERR_IO, "%s: %s: the header is not a JSON object", fn, path);
    if (strcmp(name, "__metadata__") == 0)
        return fail(TP_ERR_INVALID_ARG, "%s: \"__metadata__\" is not a tensor", fn);
    const Json *t = root.get(name);
    if (!t)
        return fail(TP_ERR_IO, "%s: %s: no tensor named \"%s\"", fn, path, name);
    const Json *dt = t->get("dtype"), *sh = t->get("shape"), *off = t->get("data_offsets");
    if (t->kind != Json::Object || !dt || dt->kind != Json::String || !sh || sh->kind != Json::Array || !off ||
        off->kind != Json::Array || off->a.size() != 2 || !off->a[0].is_int || !off->a[1].is_int)
        return fail(TP_ERR_IO, "%s: %s: malformed entry for \"%s\"", fn, path, name);
    if (dt->s == "BF16") {
        ti.dtype = TP_BF16;
        ti.es = 2;
    } else if (dt->s == "F32") {
        ti.dtype = TP_F32;
        ti.es = 4;
    } else {
        return fail(TP_ERR_UNSUPPORTED, "%s: \"%s\" has dtype %s; BF16 and F32 are supported", fn, name,
                    dt->s.c_str());
    }
    ti.ndim = (int)sh->a.size();
    if (ti.ndim < 1 || ti.ndim > 2)
        return fail(TP_ERR_UNSUPPORTED, "%s: \"%s\" has %d dimensions; 1 or 2 are supported", fn, name, ti.ndim);
    int64_t numel = 1;
    for (int d = 0; d < ti.ndim; ++d) {
        const Json &e = sh->a[d];
        if (!e.is_int || e.i < 0)
            return fail(TP_ERR_IO, "%s: %s: bad shape for \"%s\"", fn, path, name);
        if (e.i == 0 || e.i > kMaxDim)
            return fail(TP_ERR_UNSUPPORTED, "%s: \"%s\" has a dimension of %lld; 1 to 2^30 are supported", fn,
                        name, (long long)e.i);
        ti.shape[d] = e.i;
        numel *= e.i;
    }
    if (ti.ndim == 1)
        ti.shape[1] = 1;
    const int64_t begin = off->a[0].i, end = off->a[1].i;
    const int64_t data_start = 8 + (int64_t)hlen;
    if (begin < 0 || end < begin || end - begin != numel * ti.es || end > file_size - data_start)
        return fail(TP_ERR_IO, "%s: %s: data_offsets [%lld, %lld) of \"%s\" do not match its shape or the file",
                    fn, path, (long long)begin, (long long)end, name);
    ti.data_begin = data_start + begin;
    return TP_OK;
}

struct Run {
    int64_t file_off, len, dst_off;
};

// The byte runs of one rank's slice, generated in shard order.  Runs that are
// contiguous both in the file and in the shard are merged (a colwise cut of
// one block is a single run; a rowwise cut at tp 1 is one run per tensor).
class ShardRuns {
public:
    // colwise (or 1-D): one run per block, rows of row_bytes; rowwise: per row of
    // in_f elements and block, `piece[i]` elements starting at `src[i]` of the row,
    // placed at `loc[i]` of the shard row of `cols` elements.
    ShardRuns(bool rowwise, int64_t data_begin, int64_t es, int64_t row_bytes, int64_t rows, int64_t in_f,
              int64_t cols, int nb, const int64_t *piece, const int64_t *src, const int64_t *loc)
        : rowwise_(rowwise), data_begin_(data_begin), es_(es), row_bytes_(row_bytes), rows_(rowwise ? rows : 1),
          in_f_(in_f), cols_(cols), nb_(nb)
    {
        for (int i = 0; i < nb; ++i) {
            piece_[i] = piece[i];
            src_[i] = src[i];
            loc_[i] = loc[i];
        }
    }
    // The next run, or false at the end.
    bool next(Run &out)
    {
        if (!raw(out))
            return false;
        Run more;
        while (peek(more) && out.file_off + out.len == more.file_off && out.dst_off + out.len == more.dst_off) {
            out.len += more.len;
            have_peek_ = false;
        }
        return true;
    }

private:
    // The next unmerged run (from the look-ahead if there is one).
    bool raw(Run &out)
    {
        if (have_peek_) {
            out = peeked_;
            have_peek_ = false;
            return true;
        }
        while (r_ < rows_) {
            const int i = i_;
            const int64_t r = r_;
            if (++i_ == nb_) {
                i_ = 0;
                ++r_;
            }
            if (piece_[i] <= 0)
                continue;
            if (rowwise_)
                out = Run{data_begin_ + (r * in_f_ + src_[i]) * es_, piece_[i] * es_, (r * cols_ + loc_[i]) * es_};
            else
                out = Run{data_begin_ + src_[i] * row_bytes_, piece_[i] * row_bytes_, loc_[i] * row_bytes_};
            return true;
        }
        return false;
    }
    bool peek(Run &out)
    {
        if (!have_peek_)
            have_peek_ = raw(peeked_);
        out = peeked_;
        return have_peek_;
    }

    bool rowwise_;
    int64_t data_begin_, es_, row_bytes_, rows_, in_f_, cols_;
    int nb_;
    int64_t piece_[kMaxBlocks], src_[kMaxBlocks], loc_[kMaxBlocks];
    int64_t r_ = 0;
    int i_ = 0;
    Run peeked_{0, 0, 0};
    bool have_peek_ = false;
};

// Reads the pieces of one staging chunk (file offset, length, offset in
// buf; sorted by that offset, tiling [0, bytes)).  Up to kReadThreads threads
// take equal shares of the chunk's bytes, so several reads are in flight at
// once (the strided per-row reads of a rowwise cut would otherwise wait on
// the storage one at a time).  Returns false and the failing file offset on
// a read error.
bool fill_chunk(int fd, char *buf, const std::vector<Run> &pieces, int64_t bytes, int64_t *bad_off)
{
    auto read_share = [&](int64_t lo, int64_t hi, int64_t *bad) {
        // first piece that ends after lo
        const size_t k0 = (size_t)(std::upper_bound(pieces.begin(), pieces.end(), lo,
                                                    [](int64_t v, const Run &r) { return v < r.dst_off + r.len; }) -
                                   pieces.begin());
        size_t k = k0;
        // Announce every piece of the share first, so the storage sees them all at once
        // instead of one read at a time (a hint: errors are ignored).
        for (size_t j = k0; j < pieces.size() && pieces[j].dst_off < hi && pieces.size() > 1; ++j)
            (void)posix_fadvise(fd, (off_t)pieces[j].file_off, (off_t)pieces[j].len, POSIX_FADV_WILLNEED);
        for (; k < pieces.size() && pieces[k].dst_off < hi; ++k) {
            const Run &p = pieces[k];
            const int64_t a = p.dst_off > lo ? p.dst_off : lo;
            const int64_t e = p.dst_off + p.len < hi ? p.dst_off + p.len : hi;
            if (!read_full(fd, buf + a, e - a, p.file_off + (a - p.dst_off))) {
                *bad = p.file_off + (a - p.dst_off);
                return false;
            }
        }
        return true;
    };
    int nt = (int)((bytes + kMinBytesPerThread - 1) / kMinBytesPerThread);
    nt = nt < 1 ? 1 : (nt > kReadThreads ? kReadThreads : nt);
    if (nt == 1)
        return read_share(0, bytes, bad_off);
    std::vector<std::thread> th;
    std::vector<int64_t> bad((size_t)nt, -1);
    std::vector<char> ok((size_t)nt, 1);
    int handed = 1;  // shares 1 .. handed-1 run on their own threads
    try {
        for (int t = 1; t < nt; ++t) {
            th.emplace_back([&, t] { ok[t] = read_share(bytes * t / nt, bytes * (t + 1) / nt, &bad[t]); });
            handed = t + 1;
        }
    } catch (...) {
        // no more threads: this thread also reads the shares not handed out
    }
    bool mine = read_share(0, bytes / nt, &bad[0]);
    if (mine && handed < nt)
        mine = read_share(bytes * handed / nt, bytes, &bad[0]);
    ok[0] = mine;
    for (auto &x : th)
        x.join();
    for (int t = 0; t < nt; ++t)
        if (!ok[t]) {
            *bad_off = bad[t];
            return false;
        }
    return true;
}

// Copies the runs (contiguous in destination order, tiling [0, total)) into
// dst through two pinned staging buffers: while the host-to-device copy of one
// buffer runs on `stream`, the next chunk is read into the other.  Returns when
// every copy has completed.
tp_status stream_runs(const char *fn, const char *path, int fd, ShardRuns &runs, int64_t total, char *dst,
                      hipStream_t stream)
{
    const int64_t cap = total < kStageBytes ? total : kStageBytes;
    void *stage[2] = {nullptr, nullptr};
    hipEvent_t ev[2] = {nullptr, nullptr};
    bool pending[2] = {false, false};
    tp_status st = TP_OK;
    hipError_t he = hipSuccess;
    const char *what = "";

    // Staging chunks of at most cap bytes and kMaxChunkPieces pieces (file
    // offset, length, offset in the chunk), cut from the runs as they come.
    // The runs must tile [0, total) of the shard in order, so the copies never
    // leave dst: a run that does not continue where the last one ended fails.
    Run carry{0, 0, 0};     // the rest of a run that did not fit the last chunk
    int64_t planned = 0;    // shard bytes handed to chunks so far
    bool bad_plan = false;
    auto build_chunk = [&](std::vector<Run> &pieces) -> int64_t {
        pieces.clear();
        int64_t bytes = 0;
        while (!bad_plan && bytes < cap && pieces.size() < kMaxChunkPieces) {
            if (carry.len == 0) {
                if (!runs.next(carry))
                    break;
                if (carry.dst_off != planned || carry.len <= 0 || carry.len > total - planned) {
                    bad_plan = true;
                    carry.len = 0;
                    break;
                }
                planned += carry.len;
            }
            const int64_t take = carry.len < cap - bytes ? carry.len : cap - bytes;
            pieces.push_back(Run{carry.file_off, take, bytes});
            bytes += take;
            carry.file_off += take;
            carry.dst_off += take;
            carry.len -= take;
        }
        return bytes;
    };
    std::vector<Run> chunk[2];
    int64_t chunk_bytes[2] = {0, 0};
    // A chunk of a few large pieces announces the next chunk's ranges before it
    // is read, so the storage reads ahead across chunks (chunks of many small
    // pieces announce their own pieces from the reader threads instead).
    constexpr size_t kPrefetchMaxPieces = 64;
    auto prefetch = [&](const std::vector<Run> &pieces) {
        if (pieces.size() <= kPrefetchMaxPieces)
            for (const Run &p : pieces)
                (void)posix_fadvise(fd, (off_t)p.file_off, (off_t)p.len, POSIX_FADV_WILLNEED);
    };
    // Allocates staging buffer b on first use, else waits for its last copy.
    auto prepare = [&](int b) -> bool {
        if (!stage[b]) {
            he = hipHostMalloc(&stage[b], (size_t)cap, hipHostMallocDefault);
            if (he != hipSuccess) {
                stage[b] = nullptr;
                what = "hipHostMalloc";
                return false;
            }
            he = hipEventCreateWithFlags(&ev[b], hipEventDisableTiming);
            if (he != hipSuccess) {
                ev[b] = nullptr;
                what = "hipEventCreateWithFlags";
                return false;
            }
        }
        if (pending[b]) {
            he = hipEventSynchronize(ev[b]);
            pending[b] = false;
            if (he != hipSuccess) {
                what = "hipEventSynchronize";
                return false;
            }
        }
        return true;
    };

    int cur = 0;
    int64_t chunk_dst = 0;  // shard offset of the current chunk's first byte
    chunk_bytes[0] = build_chunk(chunk[0]);
    prefetch(chunk[0]);
    while (chunk_bytes[cur] > 0) {
        if (!prepare(cur))
            break;
        chunk_bytes[cur ^ 1] = build_chunk(chunk[cur ^ 1]);  // the next chunk, for its read-ahead
        prefetch(chunk[cur ^ 1]);
        int64_t bad = 0;
        if (!fill_chunk(fd, static_cast<char *>(stage[cur]), chunk[cur], chunk_bytes[cur], &bad)) {
            st = fail(TP_ERR_IO, "%s: %s: read at offset %lld failed", fn, path, (long long)bad);
            break;
        }
        he = hipMemcpyAsync(dst + chunk_dst, stage[cur], (size_t)chunk_bytes[cur], hipMemcpyHostToDevice, stream);
        if (he == hipSuccess)
            he = hipEventRecord(ev[cur], stream);
        if (he != hipSuccess) {
            what = "hipMemcpyAsync";
            break;
        }
        pending[cur] = true;
        chunk_dst += chunk_bytes[cur];
        cur ^= 1;
    }
    // Every enqueued copy must finish before its staging buffer is freed.
    for (int b = 0; b < 2; ++b) {
        if (pending[b]) {
            const hipError_t e = hipEventSynchronize(ev[b]);
            if (e != hipSuccess && he == hipSuccess) {
                he = e;
                what = "hipEventSynchronize";
            }
        }
        if (ev[b])
            (void)hipEventDestroy(ev[b]);
        if (stage[b])
            (void)hipHostFree(stage[b]);
    }
    if (st != TP_OK)
        return st;
    if (he != hipSuccess)
        return fail(TP_ERR_HIP, "%s: %s: HIP error %d (%s)", fn, what, (int)he, hipGetErrorString(he));
    if (bad_plan || chunk_dst != total)
        return fail(TP_ERR_UNSUPPORTED, "%s: internal error: byte runs cover %lld of the shard's %lld bytes", fn,
                    (long long)chunk_dst, (long long)total);
    return TP_OK;
}

struct Fd {
    int fd = -1;
    ~Fd()
    {
        if (fd >= 0)
            close(fd);
    }
};

tp_status load_shard(const char *path, const char *name, tp_style style, const int64_t *blocks, int num_blocks,
                     int tp_degree, int rank, void *dst, int64_t dst_bytes, int64_t *shard_rows,
                     int64_t *shard_cols, tp_dtype *dtype, hipStream_t stream)
{
    const char *fn = "tp_load_shard";
    if (!path || !name)
        return fail(TP_ERR_INVALID_ARG, "%s: path and name must be non-null", fn);
    if (style != TP_COLWISE && style != TP_ROWWISE && style != TP_ROWWISE_SPLIT_INPUT)
        return fail(TP_ERR_INVALID_ARG, "%s: style must be TP_COLWISE, TP_ROWWISE or TP_ROWWISE_SPLIT_INPUT", fn);
    if (tp_degree < 1)
        return fail(TP_ERR_INVALID_ARG, "%s: tp_degree=%d must be >= 1", fn, tp_degree);
    if (rank < 0 || rank >= tp_degree)
        return fail(TP_ERR_INVALID_ARG, "%s: rank=%d outside [0, %d)", fn, rank, tp_degree);
    if (!blocks && num_blocks)
        return fail(TP_ERR_INVALID_ARG, "%s: num_blocks given without blocks", fn);
    const int64_t one = 1;
    const int64_t *bl = blocks ? blocks : &one;
    const int nb = blocks ? num_blocks : 1;
    if (nb < 1 || nb > kMaxBlocks)
        return fail(TP_ERR_INVALID_ARG, "%s: num_blocks=%d must be in [1, %d]", fn, nb, kMaxBlocks);
    int64_t bsum = 0;
    for (int i = 0; i < nb; ++i) {
        if (bl[i] < 1 || bl[i] > kMaxDim)
            return fail(TP_ERR_INVALID_ARG, "%s: blocks[%d]=%lld must be a positive integer", fn, i,
                        (long long)bl[i]);
        bsum += bl[i];
    }

    Fd f;
    f.fd = open(path, O_RDONLY | O_CLOEXEC);
    if (f.fd < 0)
        return fail(TP_ERR_IO, "%s: cannot open %s: %s", fn, path, strerror(errno));
    struct stat sb;
    if (fstat(f.fd, &sb) != 0 || !S_ISREG(sb.st_mode))
        return fail(TP_ERR_IO, "%s: %s is not a readable regular file", fn, path);
    TensorInfo ti;
    tp_status s = read_tensor_info(fn, path, f.fd, (int64_t)sb.st_size, name, ti);
    if (s != TP_OK)
        return s;
    if (ti.ndim == 1 && style != TP_COLWISE)
        return fail(TP_ERR_INVALID_ARG,
                    "%s: \"%s\" is 1-D: only a colwise bias is sharded (load a rowwise bias with tp_degree 1 "
                    "and TP_COLWISE)", fn, name);

    // The sharded dimension and the packed blocks, with the slicing rules of
    // tp_plan_shard_slice: sum(blocks) divides it, each block divides by P.
    const int64_t out_f = ti.shape[0], in_f = ti.shape[1];
    const int64_t dim = ti.ndim == 1 ? out_f : (style == TP_COLWISE ? out_f : in_f);
    if (dim % bsum != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "%s: sum(blocks)=%lld does not divide the sharded dim %lld of \"%s\"", fn,
                    (long long)bsum, (long long)dim, name);
    const int64_t unit = dim / bsum;
    for (int i = 0; i < nb; ++i)
        if ((bl[i] * unit) % tp_degree != 0) {
            if (!blocks)
                return fail(TP_ERR_NOT_DIVISIBLE, "%s: tp_degree=%d does not divide the sharded dim %lld of \"%s\"",
                            fn, tp_degree, (long long)dim, name);
            return fail(TP_ERR_NOT_DIVISIBLE, "%s: packed block %d (%lld of %lld) is not divisible by tp_degree=%d",
                        fn, i, (long long)(bl[i] * unit), (long long)dim, tp_degree);
        }
    const int es = ti.es;
    int64_t rows, cols;
    if (ti.ndim == 1) {
        rows = 1;
        cols = out_f / tp_degree;
    } else {
        rows = style == TP_COLWISE ? out_f / tp_degree : out_f;
        cols = style == TP_COLWISE ? in_f : in_f / tp_degree;
    }
    if (shard_rows)
        *shard_rows = rows;
    if (shard_cols)
        *shard_cols = cols;
    if (dtype)
        *dtype = ti.dtype;
    if (!dst)
        return TP_OK;  // query only
    const int64_t total = rows * cols * es;
    if (dst_bytes < total)
        return fail(TP_ERR_INVALID_ARG, "%s: dst_bytes=%lld is below the shard's %lld bytes", fn,
                    (long long)dst_bytes, (long long)total);

    // Byte runs of the rank's slice, in shard order: block i of the sharded dim
    // holds bl[i] * unit entries, of which the rank takes `piece` starting at
    // rank * piece; in the shard it lands after the previous blocks' pieces.
    int64_t piece[kMaxBlocks], src[kMaxBlocks], loc[kMaxBlocks];
    int64_t at = 0, off = 0;
    for (int i = 0; i < nb; ++i) {
        piece[i] = bl[i] * unit / tp_degree;
        src[i] = off + rank * piece[i];
        loc[i] = at;
        at += piece[i];
        off += bl[i] * unit;
    }
    const bool rowwise = ti.ndim == 2 && style != TP_COLWISE;
    ShardRuns runs(rowwise, ti.data_begin, es, (ti.ndim == 1 ? 1 : in_f) * es, out_f, in_f, cols, nb, piece, src,
                   loc);
    return stream_runs(fn, path, f.fd, runs, total, static_cast<char *>(dst), stream);
}

}  // namespace

// The C entry point: no C++ exception may cross it.  The host-side plan (the header's
// JSON tree, the byte runs of a rowwise shard, the reader threads) can fail to allocate
// or to start for a malformed header or a very tall tensor; that is an error status.
extern "C" tp_status tp_load_shard(const char *path, const char *name, tp_style style, const int64_t *blocks,
                                   int num_blocks, int tp_degree, int rank, void *dst, int64_t dst_bytes,
                                   int64_t *shard_rows, int64_t *shard_cols, tp_dtype *dtype, hipStream_t stream)
{
    const char *fn = "tp_load_shard";
    tpl::last_error_buffer()[0] = 0;
    try {
        return load_shard(path, name, style, blocks, num_blocks, tp_degree, rank, dst, dst_bytes, shard_rows,
                          shard_cols, dtype, stream);
    } catch (const std::bad_alloc &) {
        return fail(TP_ERR_UNSUPPORTED, "%s: out of host memory while planning the read of \"%s\"", fn,
                    name ? name : "");
    } catch (const std::exception &e) {
        return fail(TP_ERR_IO, "%s: %s", fn, e.what());
    } catch (...) {
        return fail(TP_ERR_IO, "%s: unexpected exception", fn);
    }
}
