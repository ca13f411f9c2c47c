"""placeholder"""
def tpf_from_accept(mean_accept: float) -> float:
    return (mean_accept + 1.0) / 2.0
