"""placeholder"""
class VlfError(RuntimeError):
    pass
def attend(*a, **k): raise NotImplementedError
attend_into = tile_table = visible_pairs = library_path = load_library = attend
