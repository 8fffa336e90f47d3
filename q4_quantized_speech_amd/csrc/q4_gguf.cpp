// GGUF reader: the container the pages' quantised model ships in (section
// "Architecture" of "Implémentation en Rust du modèle Voxtral Mini 4B
// Realtime de Mistral pour l'exécuter dans le navigateur" names the GGUF Q4_0
// file; section "Préparation du modèle et sharding" cuts it into pieces of at
// most 512 MB that are read back as one byte stream).  Host code only: it
// parses the header, the typed metadata and the tensor table, and copies
// tensor bytes out; Q4_0 tensors come out in exactly the layout the kernels
// read.  Shards are concatenated in the order given (a plain byte split of one
// file), read with pread.
//
// Layout read (little-endian): "GGUF", uint32 version (2 or 3), uint64 tensor
// count, uint64 metadata count; metadata entries (string key, uint32 type,
// value); tensor entries (string name, uint32 n_dims, uint64 dims[n_dims] with
// dims[0] the innermost, uint32 element type, uint64 offset); padding to the
// alignment (metadata "general.alignment", default 32); the data section, each
// tensor at its offset from the section start.  Strings are a uint64 length
// and that many bytes.

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdint>
#include <cstring>
#include <memory>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/q4.h"

namespace {

enum : uint32_t {
  GT_U8 = 0, GT_I8 = 1, GT_U16 = 2, GT_I16 = 3, GT_U32 = 4, GT_I32 = 5, GT_F32 = 6, GT_BOOL = 7,
  GT_STRING = 8, GT_ARRAY = 9, GT_U64 = 10, GT_I64 = 11, GT_F64 = 12
};

constexpr uint64_t kMaxString = uint64_t(1) << 30;  // a longer string marks a corrupt file
constexpr uint32_t kMaxDims = 4;

struct Shard {
  int fd;
  uint64_t begin, size;  // position in the concatenated stream
};

struct Meta {
  std::string key;
  uint32_t type;
  uint64_t u = 0;      // integers and bools (two's complement for signed)
  double f = 0.0;      // floats
  std::string s;       // strings
  uint32_t elem = 0;   // arrays: element type and count (elements skipped)
  uint64_t count = 0;
};

struct Tensor {
  std::string name;
  uint32_t type = 0, n_dims = 0;
  int64_t dims[kMaxDims] = {1, 1, 1, 1};
  uint64_t offset = 0, nbytes = 0;
};

// Bytes of a tensor of `n` elements with innermost dimension `ne0`, for the
// element types this reader knows; 0 if unknown or malformed.
uint64_t type_bytes(uint32_t type, uint64_t n, uint64_t ne0) {
  switch (type) {
    case 0: return n * 4;                                   // F32
    case 1: return n * 2;                                   // F16
    case 30: return n * 2;                                  // BF16
    case 2: return ne0 % 32 ? 0 : n / 32 * 18;              // Q4_0
    case 8: return ne0 % 32 ? 0 : n / 32 * 34;              // Q8_0
    default: return 0;
  }
}

}  // namespace

struct q4_gguf {
  std::vector<Shard> shards;
  uint64_t total = 0;
  uint32_t version = 0;
  uint64_t alignment = 32, data_start = 0;
  std::vector<Meta> meta;
  std::vector<Tensor> tensors;
  std::unordered_map<std::string, int64_t> by_name;

  ~q4_gguf() {
    for (const Shard& s : shards)
      if (s.fd >= 0) ::close(s.fd);
  }

  // Copy [pos, pos + len) of the concatenated stream into dst.
  bool read_at(uint64_t pos, void* dst, uint64_t len) const {
    if (pos > total || len > total - pos) return false;
    char* out = static_cast<char*>(dst);
    for (const Shard& s : shards) {
      if (len == 0) break;
      if (pos >= s.begin + s.size) continue;
      uint64_t off = pos - s.begin;
      uint64_t n = s.size - off < len ? s.size - off : len;
      while (n > 0) {
        const ssize_t r = ::pread(s.fd, out, n > (uint64_t(1) << 30) ? (size_t(1) << 30) : size_t(n),
                                  static_cast<off_t>(off));
        if (r <= 0) return false;
        out += r;
        off += static_cast<uint64_t>(r);
        pos += static_cast<uint64_t>(r);
        len -= static_cast<uint64_t>(r);
        n -= static_cast<uint64_t>(r);
      }
    }
    return len == 0;
  }
};

namespace {

// Sequential reader over the stream with a small buffer.
class Cursor {
 public:
  explicit Cursor(const q4_gguf& g) : g_(g) {}
  uint64_t pos() const { return pos_; }
  bool bytes(void* dst, uint64_t n) {
    char* out = static_cast<char*>(dst);
    while (n > 0) {
      if (head_ == buf_.size()) {
        if (!fill()) return false;
      }
      const uint64_t take = buf_.size() - head_ < n ? buf_.size() - head_ : n;
      std::memcpy(out, buf_.data() + head_, take);
      head_ += take;
      out += take;
      n -= take;
      pos_ += take;
    }
    return true;
  }
  bool skip(uint64_t n) {
    const uint64_t in_buf = buf_.size() - head_;
    if (n <= in_buf) {
      head_ += n;
      pos_ += n;
      return true;
    }
    if (pos_ + n > g_.total) return false;
    pos_ += n;
    buf_.clear();
    head_ = 0;
    next_ = pos_;
    return true;
  }
  template <typename T>
  bool get(T& v) { return bytes(&v, sizeof(T)); }
  bool str(std::string& s) {
    uint64_t n = 0;
    if (!get(n) || n > kMaxString || n > g_.total - pos_) return false;
    s.resize(n);
    return bytes(&s[0], n);
  }
  uint64_t left() const { return g_.total - pos_; }

 private:
  bool fill() {
    const uint64_t n = g_.total - next_ < (uint64_t(1) << 20) ? g_.total - next_ : (uint64_t(1) << 20);
    if (n == 0) return false;
    buf_.resize(n);
    if (!g_.read_at(next_, buf_.data(), n)) return false;
    next_ += n;
    head_ = 0;
    return true;
  }
  const q4_gguf& g_;
  std::vector<char> buf_;
  uint64_t head_ = 0, pos_ = 0, next_ = 0;
};

uint64_t scalar_size(uint32_t t) {
  switch (t) {
    case GT_U8: case GT_I8: case GT_BOOL: return 1;
    case GT_U16: case GT_I16: return 2;
    case GT_U32: case GT_I32: case GT_F32: return 4;
    case GT_U64: case GT_I64: case GT_F64: return 8;
    default: return 0;
  }
}

bool read_scalar(Cursor& c, uint32_t t, Meta& m) {
  switch (t) {
    case GT_U8: { uint8_t v; if (!c.get(v)) return false; m.u = v; return true; }
    case GT_I8: { int8_t v; if (!c.get(v)) return false; m.u = static_cast<uint64_t>(int64_t(v)); return true; }
    case GT_BOOL: { uint8_t v; if (!c.get(v) || v > 1) return false; m.u = v; return true; }
    case GT_U16: { uint16_t v; if (!c.get(v)) return false; m.u = v; return true; }
    case GT_I16: { int16_t v; if (!c.get(v)) return false; m.u = static_cast<uint64_t>(int64_t(v)); return true; }
    case GT_U32: { uint32_t v; if (!c.get(v)) return false; m.u = v; return true; }
    case GT_I32: { int32_t v; if (!c.get(v)) return false; m.u = static_cast<uint64_t>(int64_t(v)); return true; }
    case GT_U64: { uint64_t v; if (!c.get(v)) return false; m.u = v; return true; }
    case GT_I64: { int64_t v; if (!c.get(v)) return false; m.u = static_cast<uint64_t>(v); return true; }
    case GT_F32: { float v; if (!c.get(v)) return false; m.f = v; return true; }
    case GT_F64: { double v; if (!c.get(v)) return false; m.f = v; return true; }
    default: return false;
  }
}

bool read_value(Cursor& c, uint32_t t, Meta& m) {
  if (t == GT_STRING) return c.str(m.s);
  if (t != GT_ARRAY) return read_scalar(c, t, m);
  if (!c.get(m.elem) || !c.get(m.count)) return false;
  if (m.elem == GT_STRING) {
    if (m.count > c.left() / 8) return false;
    for (uint64_t i = 0; i < m.count; ++i) {
      uint64_t n = 0;
      if (!c.get(n) || n > kMaxString || !c.skip(n)) return false;
    }
    return true;
  }
  const uint64_t es = scalar_size(m.elem);
  if (es == 0 || m.count > c.left() / es) return false;  // nested arrays are not used by GGUF models
  return c.skip(m.count * es);
}

bool is_int(uint32_t t) {
  return t == GT_U8 || t == GT_I8 || t == GT_U16 || t == GT_I16 || t == GT_U32 || t == GT_I32 ||
         t == GT_U64 || t == GT_I64 || t == GT_BOOL;
}

q4_status parse(q4_gguf& g) {
  Cursor c(g);
  char magic[4];
  if (!c.bytes(magic, 4) || std::memcmp(magic, "GGUF", 4) != 0) return Q4_ERR_FORMAT;
  uint64_t nt = 0, nm = 0;
  if (!c.get(g.version) || (g.version != 2 && g.version != 3)) return Q4_ERR_FORMAT;
  if (!c.get(nt) || !c.get(nm)) return Q4_ERR_FORMAT;
  if (nm > c.left() / 12 || nt > c.left() / 24) return Q4_ERR_FORMAT;  // smallest entries
  g.meta.reserve(nm);
  for (uint64_t i = 0; i < nm; ++i) {
    Meta m;
    if (!c.str(m.key) || !c.get(m.type) || !read_value(c, m.type, m)) return Q4_ERR_FORMAT;
    if (m.key == "general.alignment") {
      if (!is_int(m.type) || m.u == 0 || (m.u & (m.u - 1)) != 0) return Q4_ERR_FORMAT;
      g.alignment = m.u;
    }
    g.meta.push_back(std::move(m));
  }
  g.tensors.reserve(nt);
  for (uint64_t i = 0; i < nt; ++i) {
    Tensor t;
    if (!c.str(t.name) || !c.get(t.n_dims) || t.n_dims == 0 || t.n_dims > kMaxDims) return Q4_ERR_FORMAT;
    uint64_t n = 1;
    for (uint32_t d = 0; d < t.n_dims; ++d) {
      uint64_t v = 0;
      if (!c.get(v) || v == 0 || v > (uint64_t(1) << 40)) return Q4_ERR_FORMAT;
      if (n > (uint64_t(1) << 50) / v) return Q4_ERR_FORMAT;
      t.dims[d] = static_cast<int64_t>(v);
      n *= v;
    }
    if (!c.get(t.type) || !c.get(t.offset)) return Q4_ERR_FORMAT;
    t.nbytes = type_bytes(t.type, n, static_cast<uint64_t>(t.dims[0]));
    if (t.offset % g.alignment != 0) return Q4_ERR_FORMAT;
    if (!g.by_name.emplace(t.name, static_cast<int64_t>(g.tensors.size())).second) return Q4_ERR_FORMAT;
    g.tensors.push_back(std::move(t));
  }
  g.data_start = (c.pos() + g.alignment - 1) / g.alignment * g.alignment;
  if (g.data_start > g.total) {
    if (!g.tensors.empty()) return Q4_ERR_FORMAT;
    g.data_start = g.total;  // no tensors: the closing padding may be absent
  }
  const uint64_t data = g.total - g.data_start;
  for (const Tensor& t : g.tensors)
    if (t.nbytes != 0 && (t.offset > data || t.nbytes > data - t.offset)) return Q4_ERR_FORMAT;
  return Q4_OK;
}

const Meta* find_meta(const q4_gguf* g, const char* key) {
  if (!g || !key) return nullptr;
  for (const Meta& m : g->meta)
    if (m.key == key) return &m;
  return nullptr;
}

}  // namespace

extern "C" {

q4_status q4_gguf_open(const char* const* paths, int64_t npaths, q4_gguf** out) {
  if (!paths || !out || npaths < 1) return Q4_ERR_NULL;
  *out = nullptr;
  std::unique_ptr<q4_gguf> g(new (std::nothrow) q4_gguf());
  if (!g) return Q4_ERR_IO;
  for (int64_t i = 0; i < npaths; ++i) {
    if (!paths[i]) return Q4_ERR_NULL;
    const int fd = ::open(paths[i], O_RDONLY | O_CLOEXEC);
    if (fd < 0) return Q4_ERR_IO;
    struct stat st;
    if (::fstat(fd, &st) != 0 || st.st_size < 0) {
      ::close(fd);
      return Q4_ERR_IO;
    }
    g->shards.push_back(Shard{fd, g->total, static_cast<uint64_t>(st.st_size)});
    g->total += static_cast<uint64_t>(st.st_size);
  }
  const q4_status s = parse(*g);
  if (s != Q4_OK) return s;
  *out = g.release();
  return Q4_OK;
}

void q4_gguf_close(q4_gguf* g) { delete g; }

uint32_t q4_gguf_version(const q4_gguf* g) { return g ? g->version : 0; }

uint64_t q4_gguf_alignment(const q4_gguf* g) { return g ? g->alignment : 0; }

uint64_t q4_gguf_data_offset(const q4_gguf* g) { return g ? g->data_start : 0; }

int64_t q4_gguf_tensor_count(const q4_gguf* g) {
  return g ? static_cast<int64_t>(g->tensors.size()) : -1;
}

int64_t q4_gguf_metadata_count(const q4_gguf* g) {
  return g ? static_cast<int64_t>(g->meta.size()) : -1;
}

q4_status q4_gguf_tensor_info(const q4_gguf* g, int64_t i, const char** name, uint32_t* type,
                              uint32_t* n_dims, int64_t* dims, uint64_t* offset,
                              uint64_t* nbytes) {
  if (!g) return Q4_ERR_NULL;
  if (i < 0 || i >= static_cast<int64_t>(g->tensors.size())) return Q4_ERR_NOT_FOUND;
  const Tensor& t = g->tensors[static_cast<size_t>(i)];
  if (name) *name = t.name.c_str();
  if (type) *type = t.type;
  if (n_dims) *n_dims = t.n_dims;
  if (dims)
    for (uint32_t d = 0; d < kMaxDims; ++d) dims[d] = t.dims[d];
  if (offset) *offset = t.offset;
  if (nbytes) *nbytes = t.nbytes;
  return Q4_OK;
}

int64_t q4_gguf_find_tensor(const q4_gguf* g, const char* name) {
  if (!g || !name) return -1;
  const auto it = g->by_name.find(name);
  return it == g->by_name.end() ? -1 : it->second;
}

q4_status q4_gguf_read_tensor(const q4_gguf* g, int64_t i, void* dst, uint64_t dst_bytes) {
  if (!g || !dst) return Q4_ERR_NULL;
  if (i < 0 || i >= static_cast<int64_t>(g->tensors.size())) return Q4_ERR_NOT_FOUND;
  const Tensor& t = g->tensors[static_cast<size_t>(i)];
  if (t.nbytes == 0) return Q4_ERR_FORMAT;  // element type this reader does not size
  if (dst_bytes < t.nbytes) return Q4_ERR_WORKSPACE;
  return g->read_at(g->data_start + t.offset, dst, t.nbytes) ? Q4_OK : Q4_ERR_IO;
}

q4_status q4_gguf_metadata_key(const q4_gguf* g, int64_t i, const char** key,
                               uint32_t* value_type) {
  if (!g) return Q4_ERR_NULL;
  if (i < 0 || i >= static_cast<int64_t>(g->meta.size())) return Q4_ERR_NOT_FOUND;
  const Meta& m = g->meta[static_cast<size_t>(i)];
  if (key) *key = m.key.c_str();
  if (value_type) *value_type = m.type;
  return Q4_OK;
}

q4_status q4_gguf_metadata_int(const q4_gguf* g, const char* key, int64_t* value) {
  if (!g || !key || !value) return Q4_ERR_NULL;
  const Meta* m = find_meta(g, key);
  if (!m) return Q4_ERR_NOT_FOUND;
  if (!is_int(m->type)) return Q4_ERR_FORMAT;
  *value = static_cast<int64_t>(m->u);
  return Q4_OK;
}

q4_status q4_gguf_metadata_float(const q4_gguf* g, const char* key, double* value) {
  if (!g || !key || !value) return Q4_ERR_NULL;
  const Meta* m = find_meta(g, key);
  if (!m) return Q4_ERR_NOT_FOUND;
  if (m->type != GT_F32 && m->type != GT_F64) return Q4_ERR_FORMAT;
  *value = m->f;
  return Q4_OK;
}

q4_status q4_gguf_metadata_string(const q4_gguf* g, const char* key, const char** value,
                                  uint64_t* length) {
  if (!g || !key || !value) return Q4_ERR_NULL;
  const Meta* m = find_meta(g, key);
  if (!m) return Q4_ERR_NOT_FOUND;
  if (m->type != GT_STRING) return Q4_ERR_FORMAT;
  *value = m->s.c_str();
  if (length) *length = m->s.size();
  return Q4_OK;
}

q4_status q4_gguf_metadata_array(const q4_gguf* g, const char* key, uint32_t* elem_type,
                                 uint64_t* count) {
  if (!g || !key) return Q4_ERR_NULL;
  const Meta* m = find_meta(g, key);
  if (!m) return Q4_ERR_NOT_FOUND;
  if (m->type != GT_ARRAY) return Q4_ERR_FORMAT;
  if (elem_type) *elem_type = m->elem;
  if (count) *count = m->count;
  return Q4_OK;
}

}  // extern "C"
